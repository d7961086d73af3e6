// Internal interface of the int8-activation prefill path for Q4_K experts
// (ffn_prefill_i8.hip: the activation quantization and the i8 GEMM;
// launch_ffn_prefill_i8 in ffn_prefill.hip runs them after the tile list).
#pragma once
#include "qmoe_internal.h"

namespace qmoe {

// Workspace: the bf16 path's (h, tile list), then two int8 activation
// planes [T*k, max(H, I)], their sub-block sums [max(H, I) / 32][T*k + 256]
// and the row scales [T*k].
size_t prefill_i8_workspace_bytes(int T, int k, int H, int I);
hipError_t launch_ffn_prefill_i8(const FfnArgs& a, hipStream_t s);
hipError_t launch_i8_quant(const uint16_t* src, int K, int rows_cap, const int32_t* n_rows, const int32_t* perm,
                           int k, int8_t* a1, int8_t* a2, float* xs, int ld_xs, float* sc, hipStream_t s);
hipError_t launch_i8_gemm(bool gateup, const FfnArgs& a, const int8_t* a1, const int8_t* a2, const float* xs,
                          int ld_xs, const float* sc, const int4* tiles, const int32_t* ntiles, int max_tiles,
                          void* out, int y_dtype, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop);

}  // namespace qmoe
