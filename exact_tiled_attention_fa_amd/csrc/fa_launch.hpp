// Internal launcher interface between the C ABI (fa_api.cpp) and the kernel
// translation units.  Arguments have already been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "fa.h"
#include "fa_sched.hpp"

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Hq, Hkv, Lq, Lk, D;
  float scale;
  int causal;
  int bf16;  // 1: bfloat16, 0: float16
  int win_left = -1, win_right = -1;  // sliding window, < 0: unbounded side
  const int* cu_q = nullptr;          // packed sequences (device), or nullptr
  const int* cu_k = nullptr;
  int total_q = 0, total_k = 0;       // packed row counts
};

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const int* seqlens;
  void* o;
  float* lse;
  int B, Hq, Hkv, Lk_max, D;
  float scale;
  int num_splits;
  void* workspace;
  int bf16;
  // Paged cache (paged != 0): k/v are [num_pages, page_size, Hkv, D] pages,
  // block_table [B, max_pages]; page_size a power of two >= 16.
  int paged = 0;
  const int* block_table = nullptr;
  int page_size = 0, max_pages = 0, num_pages = 0;
  // int8 sides (paged only): codes plus float scales [num_pages, Hkv, page_size].
  int k_int8 = 0, v_int8 = 0;
  const float* k_scales = nullptr;
  const float* v_scales = nullptr;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  int B, Hq, Hkv, Lq, Lk, D;
  float scale;
  int causal;
  int win_left, win_right;
  void* workspace;
  int bf16;
  const int* cu_q = nullptr;  // packed sequences (device), or nullptr
  const int* cu_k = nullptr;
  int total_q = 0, total_k = 0;
};

struct Fp8Args {
  const void* q;   // e4m3 [B, Lq, Hq, D]; packed [total_q, Hq, D]
  const void* k;   // e4m3 [B, Lk, Hkv, D]; packed [total_k, Hkv, D]
  const void* vt;  // e4m3 [B, Hkv, D, vt_stride]; packed [Hkv, D, vt_stride]
  void* o;         // [B, Lq, Hq, D] bf16 / fp16; packed [total_q, Hq, D]
  float* lse;      // [B, Hq, Lq]; packed [Hq, total_q]
  int B, Hq, Hkv, Lq, Lk, D, vt_stride;
  float scale, q_descale, k_descale, v_descale;
  int causal;
  int win_left, win_right;
  int out_bf16;
  const int* cu_q = nullptr;  // packed sequences: offsets [B + 1], else nullptr
  const int* cu_k = nullptr;
  int total_q = 0, total_k = 0;
};

// Host-side pieces of the C ABI shared by its source files (fa_api.cpp):
// set_error records the calling thread's fa_last_error() text and returns st;
// check_decode_args validates fa_decode's arguments other than the workspace
// (FA_OK, or the status with the text recorded), before any HIP call.
fa_status set_error(fa_status st, const char* fmt, ...);
fa_status check_decode_args(const void* q, const void* k_cache, const void* v_cache,
                            const int* seqlens, const void* o, const float* lse, int B, int Hq,
                            int Hkv, int Lk_max, int D, float scale, int num_splits,
                            fa_dtype dtype);

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_fp8(const Fp8Args& a, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream);
size_t bwd_workspace_bytes(int B, int Hq, int Lq);
int bwd_padded_rows(int Lq);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
size_t decode_workspace_bytes(int B, int Hq, int D, int num_splits);

// Prefill tiling, reported by fa_info().
#ifndef FA_FWD_WAVES
#define FA_FWD_WAVES 4
#endif
constexpr int kFwdWaves = FA_FWD_WAVES;  // wavefronts per workgroup
constexpr int kFwdRowsPerWave = 32;    // query rows per wavefront
constexpr int kFwdBM = kFwdWaves * kFwdRowsPerWave;
constexpr int kDecodeKeysPerStep = 16;

}  // namespace fa
