// The W8A8 GEMM for small grids: i8_gemm.hip built with 128 x 128 tiles of
// 4 waves, two workgroups per compute unit (launch_i8_gemm_small and
// launch_f8_gemm_small, which launch_i8_gemm and launch_f8_gemm call when the
// 256 x 128 grid would fill at most half the compute units).
#define QL_I8_SMALL_TILE 1
#include "i8_gemm.hip"
