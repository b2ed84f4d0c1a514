// Host fp64 helpers of the offline calibration.
#pragma once

#include <vector>

namespace oscar {

void jacobi_eigh(std::vector<double> &A, int n, std::vector<double> &V, std::vector<double> &w);
void eigenbasis(const std::vector<double> &C, int n, std::vector<double> &U);
void compose_rotation(const std::vector<double> &U, std::vector<double> &R);
double quantile_linear(std::vector<double> &x, double p);

}  // namespace oscar
