// C ABI of libfa (declared in include/fa.h): host-side validation, error
// text and dispatch to the kernel launchers.  Nothing here touches the device
// except the launches themselves; validation failures return before any HIP
// call.
#include "fa.h"

#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "fa_launch.hpp"

namespace {

thread_local char g_err[512] = "";

fa_status fail(fa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

fa_status ok() {
  g_err[0] = '\0';
  return FA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool head_dim_supported(int D) { return D == 64 || D == 128 || D == 256; }

fa_status check_ptr(const void* p, const char* name) {
  if (!p) return fail(FA_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  if (!aligned16(p)) return fail(FA_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", name);
  return FA_OK;
}

#define FA_TRY(expr)                  \
  do {                                \
    fa_status _st = (expr);           \
    if (_st != FA_OK) return _st;     \
  } while (0)

}  // namespace

extern "C" {

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                 int Hkv, int Lq, int Lk, int D, float scale, int causal, fa_dtype dtype,
                 hipStream_t stream) {
  return fa_fwd_ex(q, k, v, o, lse, nullptr, nullptr, B, Hq, Hkv, Lq, Lk, 0, 0, D, scale, causal,
                   -1, -1, dtype, stream);
}

fa_status fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int Hq, int Hkv,
                    int Lq, int Lk, int total_q, int total_k, int D, float scale, int causal,
                    int window_left, int window_right, fa_dtype dtype, hipStream_t stream) {
  FA_TRY(check_ptr(q, "q"));
  FA_TRY(check_ptr(k, "k"));
  FA_TRY(check_ptr(v, "v"));
  FA_TRY(check_ptr(o, "o"));
  FA_TRY(check_ptr(lse, "lse"));
  const bool packed = cu_seqlens_q != nullptr || cu_seqlens_k != nullptr;
  if (packed) {
    if (!cu_seqlens_q || !cu_seqlens_k)
      return fail(FA_ERR_INVALID_ARGUMENT, "cu_seqlens_q and cu_seqlens_k must both be set or both NULL");
    if (((uintptr_t)cu_seqlens_q & 3u) || ((uintptr_t)cu_seqlens_k & 3u))
      return fail(FA_ERR_INVALID_ARGUMENT, "cu_seqlens arrays are not 4-byte aligned");
    if (total_q < 1 || total_k < 1)
      return fail(FA_ERR_INVALID_ARGUMENT, "total_q=%d and total_k=%d must be >= 1", total_q, total_k);
  }
  if (B < 1 || Hq < 1 || Hkv < 1 || Lq < 1 || Lk < 1 || D < 1)
    return fail(FA_ERR_INVALID_ARGUMENT,
                "sizes must be >= 1 (B=%d Hq=%d Hkv=%d Lq=%d Lk=%d D=%d)", B, Hq, Hkv, Lq, Lk, D);
  if (Hq % Hkv != 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (!isfinite(scale)) return fail(FA_ERR_INVALID_ARGUMENT, "scale is not finite");
  if (dtype != FA_F16 && dtype != FA_BF16)
    return fail(FA_ERR_UNSUPPORTED, "dtype %d is not FA_F16 or FA_BF16", (int)dtype);
  if (!head_dim_supported(D))
    return fail(FA_ERR_UNSUPPORTED, "head_dim %d not in {64, 128, 256}", D);
  // The kernel addresses a K/V tile with 32-bit byte offsets: 64 rows of
  // Hkv * D elements must stay below 4 GiB.
  if ((long long)Hkv * D >= (1LL << 25))
    return fail(FA_ERR_INVALID_ARGUMENT, "Hkv * D = %lld must be < 2^25", (long long)Hkv * D);
  const long long nqt = ((long long)Lq + fa::kFwdBM - 1) / fa::kFwdBM;
  if (nqt * B * Hq > 0x7fffffffLL)
    return fail(FA_ERR_INVALID_ARGUMENT, "grid too large (Lq/%d * B * Hq > 2^31-1)", fa::kFwdBM);
  const long long rows_q = packed ? (long long)total_q : (long long)B * Lq;
  const long long rows_k = packed ? (long long)total_k : (long long)B * Lk;
  if (rows_q * Hq > 0x7fffffffLL || rows_k * Hkv > 0x7fffffffLL)
    return fail(FA_ERR_INVALID_ARGUMENT, "B*L*H (rows * heads) exceeds 2^31-1");
  // Window bounds are evaluated in 32-bit arithmetic: a side at least as wide
  // as every sequence is the same as no bound, and with a window the query
  // plus key rows are kept below 2^30 so that i + (Lk - Lq) -/+ window fits.
  const long long span = rows_q + rows_k;
  const bool windowed = window_left >= 0 || window_right >= 0;
  if (windowed && span > (1LL << 30))
    return fail(FA_ERR_INVALID_ARGUMENT, "windowed attention needs query + key rows <= 2^30");

  fa::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, scale, causal ? 1 : 0,
                dtype == FA_BF16 ? 1 : 0};
  a.win_left = (window_left < 0 || window_left >= span) ? -1 : window_left;
  a.win_right = (window_right < 0 || window_right >= span) ? -1 : window_right;
  a.cu_q = packed ? cu_seqlens_q : nullptr;
  a.cu_k = packed ? cu_seqlens_k : nullptr;
  a.total_q = packed ? total_q : 0;
  a.total_k = packed ? total_k : 0;
  hipError_t e = fa::launch_fwd(a, stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "attention forward launch failed: %s", hipGetErrorString(e));
  return ok();
}

fa_status fa_fwd_fp8_ex(const void* q8, const void* k8, const void* vt8, void* o, float* lse,
                        const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int Hq, int Hkv,
                        int Lq, int Lk, int total_q, int total_k, int D, int vt_stride,
                        float scale, float q_descale, float k_descale, float v_descale,
                        int causal, int window_left, int window_right, fa_dtype out_dtype,
                        hipStream_t stream) {
  FA_TRY(check_ptr(q8, "q8"));
  FA_TRY(check_ptr(k8, "k8"));
  FA_TRY(check_ptr(vt8, "vt8"));
  FA_TRY(check_ptr(o, "o"));
  FA_TRY(check_ptr(lse, "lse"));
  const bool packed = cu_seqlens_q != nullptr || cu_seqlens_k != nullptr;
  if (packed) {
    if (!cu_seqlens_q || !cu_seqlens_k)
      return fail(FA_ERR_INVALID_ARGUMENT, "cu_seqlens_q and cu_seqlens_k must both be set or both NULL");
    if (((uintptr_t)cu_seqlens_q & 3u) || ((uintptr_t)cu_seqlens_k & 3u))
      return fail(FA_ERR_INVALID_ARGUMENT, "cu_seqlens arrays are not 4-byte aligned");
    if (total_q < 1 || total_k < 1)
      return fail(FA_ERR_INVALID_ARGUMENT, "total_q=%d and total_k=%d must be >= 1", total_q, total_k);
  }
  if (B < 1 || Hq < 1 || Hkv < 1 || Lq < 1 || Lk < 1 || D < 1)
    return fail(FA_ERR_INVALID_ARGUMENT,
                "sizes must be >= 1 (B=%d Hq=%d Hkv=%d Lq=%d Lk=%d D=%d)", B, Hq, Hkv, Lq, Lk, D);
  if (Hq % Hkv != 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (!isfinite(scale)) return fail(FA_ERR_INVALID_ARGUMENT, "scale is not finite");
  if (!(isfinite(q_descale) && isfinite(k_descale) && isfinite(v_descale) && q_descale > 0.f &&
        k_descale > 0.f && v_descale > 0.f))
    return fail(FA_ERR_INVALID_ARGUMENT, "descales must be finite and > 0");
  if (out_dtype != FA_F16 && out_dtype != FA_BF16)
    return fail(FA_ERR_UNSUPPORTED, "dtype %d is not FA_F16 or FA_BF16", (int)out_dtype);
  if (!head_dim_supported(D))
    return fail(FA_ERR_UNSUPPORTED, "fp8 head_dim %d not in {64, 128, 256}", D);
  // Key tiles read 64 columns of V^T from a 16-aligned start: dense rows hold
  // Lk keys (padded to 64), packed rows total_k keys plus 64 columns of
  // padding.
  const long long vt_need = packed ? (long long)total_k + 64 : (long long)Lk;
  if (vt_stride % 64 != 0 || vt_stride < vt_need)
    return fail(FA_ERR_INVALID_ARGUMENT, "vt_stride=%d must be a multiple of 64 and >= %lld",
                vt_stride, vt_need);
  if ((long long)D * vt_stride >= (1LL << 32))
    return fail(FA_ERR_INVALID_ARGUMENT, "D * vt_stride must be < 2^32");
  if ((long long)Hkv * D >= (1LL << 25) || (long long)Hq * D >= (1LL << 25))
    return fail(FA_ERR_INVALID_ARGUMENT, "Hq * D and Hkv * D must be < 2^25");
  const long long rows_q = packed ? (long long)total_q : (long long)B * Lq;
  const long long rows_k = packed ? (long long)total_k : (long long)B * Lk;
  if (rows_q * Hq > 0x7fffffffLL || rows_k * Hkv > 0x7fffffffLL)
    return fail(FA_ERR_INVALID_ARGUMENT, "B*L*H exceeds 2^31-1 rows");
  // at D = 256 two workgroups share each query tile (128 output dims each)
  if (((long long)Lq + 127) / 128 * B * Hq * (D / 128 > 1 ? 2 : 1) > 0x7fffffffLL)
    return fail(FA_ERR_INVALID_ARGUMENT, "grid too large (Lq/128 * B * Hq > 2^31-1)");
  const long long span = rows_q + rows_k;
  const bool windowed = window_left >= 0 || window_right >= 0;
  if (windowed && span > (1LL << 30))
    return fail(FA_ERR_INVALID_ARGUMENT, "windowed attention needs query + key rows <= 2^30");
  fa::Fp8Args a{q8, k8, vt8, o, lse, B, Hq, Hkv, Lq, Lk, D, vt_stride, scale, q_descale,
                k_descale, v_descale, causal ? 1 : 0,
                (window_left < 0 || window_left >= span) ? -1 : window_left,
                (window_right < 0 || window_right >= span) ? -1 : window_right,
                out_dtype == FA_BF16 ? 1 : 0};
  a.cu_q = packed ? cu_seqlens_q : nullptr;
  a.cu_k = packed ? cu_seqlens_k : nullptr;
  a.total_q = packed ? total_q : 0;
  a.total_k = packed ? total_k : 0;
  hipError_t e = fa::launch_fwd_fp8(a, stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "fa_fwd_fp8 launch failed: %s", hipGetErrorString(e));
  return ok();
}

fa_status fa_fwd_fp8(const void* q8, const void* k8, const void* vt8, void* o, float* lse, int B,
                     int Hq, int Hkv, int Lq, int Lk, int D, int vt_stride, float scale,
                     float q_descale, float k_descale, float v_descale, int causal,
                     int window_left, int window_right, fa_dtype out_dtype, hipStream_t stream) {
  return fa_fwd_fp8_ex(q8, k8, vt8, o, lse, nullptr, nullptr, B, Hq, Hkv, Lq, Lk, 0, 0, D,
                       vt_stride, scale, q_descale, k_descale, v_descale, causal, window_left,
                       window_right, out_dtype, stream);
}

size_t fa_decode_workspace_size(int B, int Hq, int D, int num_splits) {
  if (B < 1 || Hq < 1 || D < 1 || num_splits < 1 || num_splits > 64) return 0;
  return fa::decode_workspace_bytes(B, Hq, D, num_splits);
}

}  // extern "C"

namespace fa {

fa_status set_error(fa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

fa_status check_decode_args(const void* q, const void* k_cache, const void* v_cache,
                            const int* seqlens, const void* o, const float* lse, int B, int Hq,
                            int Hkv, int Lk_max, int D, float scale, int num_splits,
                            fa_dtype dtype) {
  FA_TRY(check_ptr(q, "q"));
  FA_TRY(check_ptr(k_cache, "k_cache"));
  FA_TRY(check_ptr(v_cache, "v_cache"));
  if (!seqlens) return fail(FA_ERR_INVALID_ARGUMENT, "seqlens is NULL");
  if (((uintptr_t)seqlens & 3u) != 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "seqlens is not 4-byte aligned");
  FA_TRY(check_ptr(o, "o"));
  FA_TRY(check_ptr(lse, "lse"));
  if (B < 1 || Hq < 1 || Hkv < 1 || Lk_max < 1 || D < 1)
    return fail(FA_ERR_INVALID_ARGUMENT, "sizes must be >= 1 (B=%d Hq=%d Hkv=%d Lk_max=%d D=%d)",
                B, Hq, Hkv, Lk_max, D);
  if (Hq % Hkv != 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (num_splits < 1 || num_splits > 64)
    return fail(FA_ERR_INVALID_ARGUMENT, "num_splits=%d not in [1, 64]", num_splits);
  if (!isfinite(scale)) return fail(FA_ERR_INVALID_ARGUMENT, "scale is not finite");
  if (dtype != FA_F16 && dtype != FA_BF16)
    return fail(FA_ERR_UNSUPPORTED, "dtype %d is not FA_F16 or FA_BF16", (int)dtype);
  if (!head_dim_supported(D))
    return fail(FA_ERR_UNSUPPORTED, "head_dim %d not in {64, 128, 256}", D);
  if ((long long)B * Lk_max * Hkv > 0x7fffffffLL)
    return fail(FA_ERR_INVALID_ARGUMENT, "B*Lk_max*Hkv exceeds 2^31-1 rows");
  if ((long long)Hkv * ((Hq / Hkv + 15) / 16) > 65535 || B > 65535)
    return fail(FA_ERR_INVALID_ARGUMENT, "grid too large (B or Hq exceeds 65535)");
  return FA_OK;
}

}  // namespace fa

extern "C" {

fa_status fa_decode(const void* q, const void* k_cache, const void* v_cache, const int* seqlens,
                    void* o, float* lse, int B, int Hq, int Hkv, int Lk_max, int D, float scale,
                    int num_splits, void* workspace, size_t workspace_bytes, fa_dtype dtype,
                    hipStream_t stream) {
  FA_TRY(fa::check_decode_args(q, k_cache, v_cache, seqlens, o, lse, B, Hq, Hkv, Lk_max, D, scale,
                               num_splits, dtype));
  FA_TRY(check_ptr(workspace, "workspace"));
  const size_t need = fa::decode_workspace_bytes(B, Hq, D, num_splits);
  if (workspace_bytes < need)
    return fail(FA_ERR_INVALID_ARGUMENT, "workspace has %zu bytes, needs %zu", workspace_bytes,
                need);

  fa::DecodeArgs a{q, k_cache, v_cache, seqlens, o, lse, B, Hq, Hkv, Lk_max, D, scale,
                   num_splits, workspace, dtype == FA_BF16 ? 1 : 0};
  hipError_t e = fa::launch_decode(a, stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "fa_decode launch failed: %s", hipGetErrorString(e));
  return ok();
}

fa_status fa_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                          const float* k_scales, const float* v_scales, const int* block_table,
                          const int* seqlens, void* o, float* lse, int B, int Hq, int Hkv, int D,
                          int num_pages, int page_size, int max_pages, float scale,
                          int num_splits, fa_kv_format k_format, fa_kv_format v_format,
                          void* workspace, size_t workspace_bytes, fa_dtype dtype,
                          hipStream_t stream) {
  FA_TRY(check_ptr(q, "q"));
  FA_TRY(check_ptr(k_pages, "k_pages"));
  FA_TRY(check_ptr(v_pages, "v_pages"));
  FA_TRY(check_ptr(o, "o"));
  FA_TRY(check_ptr(lse, "lse"));
  FA_TRY(check_ptr(workspace, "workspace"));
  if (!block_table) return fail(FA_ERR_INVALID_ARGUMENT, "block_table is NULL");
  if (!seqlens) return fail(FA_ERR_INVALID_ARGUMENT, "seqlens is NULL");
  if (((uintptr_t)block_table & 3u) || ((uintptr_t)seqlens & 3u))
    return fail(FA_ERR_INVALID_ARGUMENT, "block_table and seqlens must be 4-byte aligned");
  if ((k_format != FA_KV_NATIVE && k_format != FA_KV_INT8) ||
      (v_format != FA_KV_NATIVE && v_format != FA_KV_INT8))
    return fail(FA_ERR_UNSUPPORTED, "kv formats %d/%d are not FA_KV_NATIVE or FA_KV_INT8",
                (int)k_format, (int)v_format);
  if (k_format == FA_KV_NATIVE && v_format == FA_KV_INT8)
    return fail(FA_ERR_UNSUPPORTED, "int8 values need int8 keys");
  const bool k8 = k_format == FA_KV_INT8, v8 = v_format == FA_KV_INT8;
  if (k8 && (!k_scales || !aligned16(k_scales)))
    return fail(FA_ERR_INVALID_ARGUMENT, "k_scales must be a 16-byte aligned pointer for int8 keys");
  if (v8 && (!v_scales || !aligned16(v_scales)))
    return fail(FA_ERR_INVALID_ARGUMENT, "v_scales must be a 16-byte aligned pointer for int8 values");
  if (B < 1 || Hq < 1 || Hkv < 1 || D < 1 || num_pages < 1 || max_pages < 1)
    return fail(FA_ERR_INVALID_ARGUMENT,
                "sizes must be >= 1 (B=%d Hq=%d Hkv=%d D=%d num_pages=%d max_pages=%d)", B, Hq,
                Hkv, D, num_pages, max_pages);
  if (page_size < 16 || page_size > 65536 || (page_size & (page_size - 1)))
    return fail(FA_ERR_INVALID_ARGUMENT, "page_size=%d is not a power of two in [16, 65536]",
                page_size);
  if (Hq % Hkv != 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (num_splits < 1 || num_splits > 64)
    return fail(FA_ERR_INVALID_ARGUMENT, "num_splits=%d not in [1, 64]", num_splits);
  if (!isfinite(scale)) return fail(FA_ERR_INVALID_ARGUMENT, "scale is not finite");
  if (dtype != FA_F16 && dtype != FA_BF16)
    return fail(FA_ERR_UNSUPPORTED, "dtype %d is not FA_F16 or FA_BF16", (int)dtype);
  if (!head_dim_supported(D))
    return fail(FA_ERR_UNSUPPORTED, "head_dim %d not in {64, 128, 256}", D);
  if ((long long)max_pages * page_size > 0x7fffffffLL)
    return fail(FA_ERR_INVALID_ARGUMENT, "max_pages * page_size exceeds 2^31-1");
  if ((long long)B * max_pages > 0x7fffffffLL)
    return fail(FA_ERR_INVALID_ARGUMENT, "B * max_pages exceeds 2^31-1");
  if ((long long)Hkv * ((Hq / Hkv + 15) / 16) > 65535 || B > 65535)
    return fail(FA_ERR_INVALID_ARGUMENT, "grid too large (B or Hq exceeds 65535)");
  const size_t need = fa::decode_workspace_bytes(B, Hq, D, num_splits);
  if (workspace_bytes < need)
    return fail(FA_ERR_INVALID_ARGUMENT, "workspace has %zu bytes, needs %zu", workspace_bytes,
                need);

  fa::DecodeArgs a{q, k_pages, v_pages, seqlens, o, lse, B, Hq, Hkv, 0, D, scale,
                   num_splits, workspace, dtype == FA_BF16 ? 1 : 0};
  a.paged = 1;
  a.block_table = block_table;
  a.page_size = page_size;
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  a.k_int8 = k8 ? 1 : 0;
  a.v_int8 = v8 ? 1 : 0;
  a.k_scales = k8 ? k_scales : nullptr;
  a.v_scales = v8 ? v_scales : nullptr;
  hipError_t e = fa::launch_decode(a, stream);
  if (e != hipSuccess)
    return fail(FA_ERR_HIP, "fa_decode_paged launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t fa_bwd_workspace_size(int B, int Hq, int Lq) {
  if (B < 1 || Hq < 1 || Lq < 1) return 0;
  return fa::bwd_workspace_bytes(B, Hq, Lq);
}

fa_status fa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, void* dq, void* dk, void* dv, const int* cu_seqlens_q,
                    const int* cu_seqlens_k, int B, int Hq, int Hkv, int Lq, int Lk, int total_q,
                    int total_k, int D, float scale, int causal, int window_left,
                    int window_right, void* workspace, size_t workspace_bytes, fa_dtype dtype,
                    hipStream_t stream) {
  FA_TRY(check_ptr(q, "q"));
  FA_TRY(check_ptr(k, "k"));
  FA_TRY(check_ptr(v, "v"));
  FA_TRY(check_ptr(o, "o"));
  FA_TRY(check_ptr(dout, "dout"));
  FA_TRY(check_ptr(lse, "lse"));
  FA_TRY(check_ptr(dq, "dq"));
  FA_TRY(check_ptr(dk, "dk"));
  FA_TRY(check_ptr(dv, "dv"));
  FA_TRY(check_ptr(workspace, "workspace"));
  const bool packed = cu_seqlens_q != nullptr || cu_seqlens_k != nullptr;
  if (packed) {
    if (!cu_seqlens_q || !cu_seqlens_k)
      return fail(FA_ERR_INVALID_ARGUMENT, "cu_seqlens_q and cu_seqlens_k must both be set or both NULL");
    if (((uintptr_t)cu_seqlens_q & 3u) || ((uintptr_t)cu_seqlens_k & 3u))
      return fail(FA_ERR_INVALID_ARGUMENT, "cu_seqlens arrays are not 4-byte aligned");
    if (total_q < 1 || total_k < 1)
      return fail(FA_ERR_INVALID_ARGUMENT, "total_q=%d and total_k=%d must be >= 1", total_q, total_k);
  }
  if (B < 1 || Hq < 1 || Hkv < 1 || Lq < 1 || Lk < 1 || D < 1)
    return fail(FA_ERR_INVALID_ARGUMENT,
                "sizes must be >= 1 (B=%d Hq=%d Hkv=%d Lq=%d Lk=%d D=%d)", B, Hq, Hkv, Lq, Lk, D);
  if (Hq % Hkv != 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (!isfinite(scale)) return fail(FA_ERR_INVALID_ARGUMENT, "scale is not finite");
  if (dtype != FA_F16 && dtype != FA_BF16)
    return fail(FA_ERR_UNSUPPORTED, "dtype %d is not FA_F16 or FA_BF16", (int)dtype);
  if (!head_dim_supported(D))
    return fail(FA_ERR_UNSUPPORTED, "head_dim %d not in {64, 128, 256}", D);
  if ((long long)Hq * D >= (1LL << 25) || (long long)Hkv * D >= (1LL << 25))
    return fail(FA_ERR_INVALID_ARGUMENT, "Hq * D and Hkv * D must be < 2^25");
  const long long rows_q = packed ? (long long)total_q : (long long)B * Lq;
  const long long rows_k = packed ? (long long)total_k : (long long)B * Lk;
  if (rows_q * Hq > 0x7fffffffLL || rows_k * Hkv > 0x7fffffffLL ||
      (long long)B * Lq * Hq > 0x7fffffffLL)
    return fail(FA_ERR_INVALID_ARGUMENT, "B*L*H (rows * heads) exceeds 2^31-1");
  if (((long long)Lq + 127) / 128 * B * Hq > 0x7fffffffLL ||
      ((long long)Lk + 63) / 64 * B * Hkv > 0x7fffffffLL)
    return fail(FA_ERR_INVALID_ARGUMENT, "grid too large (Lq/128 * B * Hq or Lk/64 * B * Hkv > 2^31-1)");
  const long long span = rows_q + rows_k;
  const bool windowed = window_left >= 0 || window_right >= 0;
  if (windowed && span > (1LL << 30))
    return fail(FA_ERR_INVALID_ARGUMENT, "windowed attention needs query + key rows <= 2^30");
  const size_t need = fa::bwd_workspace_bytes(B, Hq, Lq);
  if (workspace_bytes < need)
    return fail(FA_ERR_INVALID_ARGUMENT, "workspace has %zu bytes, needs %zu", workspace_bytes,
                need);

  fa::BwdArgs a{q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, Lq, Lk, D, scale, causal ? 1 : 0,
                (window_left < 0 || window_left >= span) ? -1 : window_left,
                (window_right < 0 || window_right >= span) ? -1 : window_right, workspace,
                dtype == FA_BF16 ? 1 : 0};
  a.cu_q = packed ? cu_seqlens_q : nullptr;
  a.cu_k = packed ? cu_seqlens_k : nullptr;
  a.total_q = packed ? total_q : 0;
  a.total_k = packed ? total_k : 0;
  hipError_t e = fa::launch_bwd(a, stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "fa_bwd launch failed: %s", hipGetErrorString(e));
  return ok();
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Lq,
                 int Lk, int D, float scale, int causal, int window_left, int window_right,
                 void* workspace, size_t workspace_bytes, fa_dtype dtype, hipStream_t stream) {
  return fa_bwd_ex(q, k, v, o, dout, lse, dq, dk, dv, nullptr, nullptr, B, Hq, Hkv, Lq, Lk, 0, 0,
                   D, scale, causal, window_left, window_right, workspace, workspace_bytes, dtype,
                   stream);
}

const char* fa_last_error(void) { return g_err; }

const char* fa_info(void) {
  return "arch=gfx950; head_dims={64,128,256}; dtypes={f16,bf16}; "
         "fwd: 4 wave64 x 32 query rows per workgroup (BM=128; at D=256 8 wave64, two per "
         "row slice splitting the head dims), 32-key tiles, "
         "mfma_f32_32x32x16, LDS-direct K/V with transpose reads, causal/window tile "
         "skip, block-diagonal packing, GQA; "
         "bwd: dQ query-major, dK/dV key-major in pairs of waves, dense and packed, D={64,128,256}; "
         "decode: split-KV, 4 wave64 per (chunk, kv head, 16 heads, sequence), 16-key steps, "
         "mfma_f32_16x16x32 + 16x16x16, logsumexp combine, paged and int8 KV caches; "
         "fp8 fwd: e4m3 mfma_scale_f32_32x32x64_f8f6f4, D={64,128,256}; "
         "version=0.5.0";
}

}  // extern "C"
