// Host fp64 helpers of the offline calibration.
#pragma once

#include <vector>

namespace oscar {

// U: columns of V reordered by descending w, each with its largest-|entry| positive
void sorted_basis(const std::vector<double> &V, const std::vector<double> &w, int n, std::vector<double> &U);
void compose_rotation(const std::vector<double> &U, std::vector<double> &R);
double quantile_linear(std::vector<double> &x, double p);

}  // namespace oscar
