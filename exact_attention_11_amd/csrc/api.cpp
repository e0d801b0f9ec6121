// C ABI of libfattn: argument validation and kernel dispatch.
//
// Every check happens on the host before anything is launched; an invalid call
// returns a status and leaves a message in a thread-local buffer.  No
// exception crosses the ABI and no device memory is allocated here.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "fattn.h"
#include "launch.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return FATTN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(FATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr float kLog2e = 1.4426950408889634f;

// Shared shape checks of the dense forward calls.
int check_dense(const char* fn, const void* q, const void* k, const void* v, const void* o, const float* lse, int B,
                int H, int Hkv, int N, float scale, int causal) {
  if (B < 0 || N < 0) return fail(FATTN_ERR_INVALID_ARG, "%s: B and N must be >= 0 (got B=%d N=%d)", fn, B, N);
  if (H < 1 || Hkv < 1) return fail(FATTN_ERR_INVALID_ARG, "%s: H and Hkv must be >= 1 (got H=%d Hkv=%d)", fn, H, Hkv);
  if (H % Hkv != 0) return fail(FATTN_ERR_INVALID_ARG, "%s: H=%d is not a multiple of Hkv=%d", fn, H, Hkv);
  if (causal != 0 && causal != 1) return fail(FATTN_ERR_INVALID_ARG, "%s: causal must be 0 or 1 (got %d)", fn, causal);
  if (!std::isfinite(scale) || scale < 0.f)
    return fail(FATTN_ERR_INVALID_ARG, "%s: scale must be finite and >= 0 (got %g)", fn, (double)scale);
  if (B == 0 || N == 0) return FATTN_OK;
  if (!q || !k || !v || !o) return fail(FATTN_ERR_INVALID_ARG, "%s: q, k, v and o must be non-null", fn);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (lse && !aligned16(lse)))
    return fail(FATTN_ERR_INVALID_ARG, "%s: tensor pointers must be 16-byte aligned", fn);
  const double rows = (double)B * H * N;
  if (rows > 2147483647.0) return fail(FATTN_ERR_INVALID_ARG, "%s: B*H*N too large", fn);
  return FATTN_OK;
}

}  // namespace

extern "C" {

const char* fattn_status_string(int status) {
  switch (status) {
    case FATTN_OK: return "FATTN_OK";
    case FATTN_ERR_INVALID_ARG: return "FATTN_ERR_INVALID_ARG";
    case FATTN_ERR_UNSUPPORTED: return "FATTN_ERR_UNSUPPORTED";
    case FATTN_ERR_HIP: return "FATTN_ERR_HIP";
    case FATTN_ERR_INTERNAL: return "FATTN_ERR_INTERNAL";
    default: return "FATTN_ERR_UNKNOWN";
  }
}

const char* fattn_last_error(void) { return g_last_error.c_str(); }

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv, int N, int d,
             float scale, int causal, void* stream) {
  int st = check_dense("attn_fwd", q, k, v, o, lse, B, H, Hkv, N, scale, causal);
  if (st != FATTN_OK) return st;
  if (d != 64 && d != 128 && d != 256)
    return fail(FATTN_ERR_UNSUPPORTED, "attn_fwd: d=%d not supported (64, 128 or 256)", d);
  if (B == 0 || N == 0) return ok();
  // K/V rows of one head are addressed with 32-bit byte offsets
  if ((double)N * d * 2 >= 4294967296.0) return fail(FATTN_ERR_INVALID_ARG, "attn_fwd: N*d too large for one head");
  fattn::TileArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.offsets = nullptr;
  a.B = B;
  a.H = H;
  a.Hkv = Hkv;
  a.N = N;
  a.d = d;
  // scale == 0 runs as the smallest normal scale: for any finite score s,
  // s * FLT_MIN * log2(e) rounds away against 1 in exp2, so every visible
  // weight is exactly 1 (the scale-0 result), and masked scores (-inf) still
  // give weight exactly 0.
  a.c = std::fmax(scale * kLog2e, FLT_MIN);
  a.inv_n = 1.f;
  a.causal = causal;
  a.epi = fattn::Epilogue::Softmax;
  return hip_status(fattn::launch_tile_bf16(a, static_cast<hipStream_t>(stream)), "attn_fwd launch");
}

int attn_fwd_f32(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv, int N, int d,
                 float scale, int causal, void* stream) {
  int st = check_dense("attn_fwd_f32", q, k, v, o, lse, B, H, Hkv, N, scale, causal);
  if (st != FATTN_OK) return st;
  if (d != 64) return fail(FATTN_ERR_UNSUPPORTED, "attn_fwd_f32: d=%d not supported (64)", d);
  if (B == 0 || N == 0) return ok();
  fattn::F32Args a{};
  a.q = static_cast<const float*>(q);
  a.k = static_cast<const float*>(k);
  a.v = static_cast<const float*>(v);
  a.o = static_cast<float*>(o);
  a.lse = lse;
  a.B = B;
  a.H = H;
  a.Hkv = Hkv;
  a.N = N;
  a.d = d;
  a.c = scale * kLog2e;
  a.causal = causal;
  return hip_status(fattn::launch_prefill_f32(a, static_cast<hipStream_t>(stream)), "attn_fwd_f32 launch");
}

int attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, const float* descale_q,
                 const float* descale_k, const float* descale_v, int B, int H, int Hkv, int N, int d, float scale,
                 int causal, void* stream) {
  const char* fn = "attn_fwd_fp8";
  int st = check_dense(fn, q, k, v, o, lse, B, H, Hkv, N, scale, causal);
  if (st != FATTN_OK) return st;
  if (d != 128) return fail(FATTN_ERR_UNSUPPORTED, "%s: d=%d not supported (128)", fn, d);
  if (B == 0 || N == 0) return ok();
  if (!descale_q || !descale_k || !descale_v)
    return fail(FATTN_ERR_INVALID_ARG, "%s: descale_q, descale_k and descale_v must be non-null", fn);
  if ((double)N * d >= 4294967296.0) return fail(FATTN_ERR_INVALID_ARG, "%s: N*d too large for one head", fn);
  fattn::Fp8Args a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.descale_q = descale_q;
  a.descale_k = descale_k;
  a.descale_v = descale_v;
  a.B = B;
  a.H = H;
  a.Hkv = Hkv;
  a.N = N;
  a.d = d;
  a.c = scale * kLog2e;
  a.causal = causal;
  return hip_status(fattn::launch_tile_fp8(a, static_cast<hipStream_t>(stream)), "attn_fwd_fp8 launch");
}

size_t attn_decode_workspace_bytes(int B, int H, int d, int num_splits) {
  if (B < 0 || H < 1 || d < 1 || num_splits < 0 || num_splits > 64) return 0;
  // the automatic count of either entry point is at most 64 splits
  const int s = num_splits == 0 ? 64 : num_splits;
  const size_t bytes = (size_t)H * B * (s + 1) * ((size_t)d + 1) * sizeof(float);
  return (bytes + 255) / 256 * 256;
}

}  // extern "C"

namespace {

// Validation shared by attn_decode and attn_decode_noalloc: every argument
// except the workspace; on success `a` is filled except part_o / part_lse and
// `need` holds the workspace bytes the call uses.  `*done` is set when the
// call has nothing to launch (B == 0).
int prepare_decode(const char* fn, const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* seqlens_k, void* o, float* lse, int B, int H, int Hkv, int Lmax, int d, float scale,
                   int num_splits, fattn::DecodeArgs& a, size_t& need, bool* done) {
  *done = false;
  if (B < 0) return fail(FATTN_ERR_INVALID_ARG, "%s: B must be >= 0 (got %d)", fn, B);
  if (H < 1 || Hkv < 1) return fail(FATTN_ERR_INVALID_ARG, "%s: H and Hkv must be >= 1", fn);
  if (H % Hkv != 0) return fail(FATTN_ERR_INVALID_ARG, "%s: H=%d is not a multiple of Hkv=%d", fn, H, Hkv);
  if (Lmax < 1) return fail(FATTN_ERR_INVALID_ARG, "%s: Lmax must be >= 1 (got %d)", fn, Lmax);
  if (!std::isfinite(scale) || scale < 0.f)
    return fail(FATTN_ERR_INVALID_ARG, "%s: scale must be finite and >= 0 (got %g)", fn, (double)scale);
  if (num_splits < 0 || num_splits > 64)
    return fail(FATTN_ERR_INVALID_ARG, "%s: num_splits must be 0 (auto) or 1..64 (got %d)", fn, num_splits);
  const int G = H / Hkv;
  if (d != 128) return fail(FATTN_ERR_UNSUPPORTED, "%s: d=%d not supported (128)", fn, d);
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16 && G != 32)
    return fail(FATTN_ERR_UNSUPPORTED, "%s: H/Hkv=%d not supported (1, 2, 4, 8, 16 or 32)", fn, G);
  if (B == 0) {
    *done = true;
    return FATTN_OK;
  }
  if (!q || !k_cache || !v_cache || !seqlens_k || !o)
    return fail(FATTN_ERR_INVALID_ARG, "%s: q, caches, seqlens_k and o must be non-null", fn);
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) || (lse && !aligned16(lse)))
    return fail(FATTN_ERR_INVALID_ARG, "%s: tensor pointers must be 16-byte aligned", fn);
  if ((double)B * Hkv * Lmax * d > 9.0e15) return fail(FATTN_ERR_INVALID_ARG, "%s: cache too large", fn);
  const int splits = num_splits == 0 ? fattn::decode_auto_splits(B, Hkv, Lmax, false) : num_splits;
  // a work item holds at most ceil(ceil(Lmax / 32) / splits) blocks of 32 keys
  // of 256 bytes each per kv head; its byte offsets are 32-bit
  const double item_bytes = std::ceil(std::ceil(Lmax / 32.0) / splits) * 32.0 * (d * 2);
  if (item_bytes >= 4294967296.0)
    return fail(FATTN_ERR_UNSUPPORTED, "%s: a work item of %.0f bytes per kv head passes 32-bit offsets; use more splits",
                fn, item_bytes);
  need = attn_decode_workspace_bytes(B, H, d, splits);
  a = fattn::DecodeArgs{};
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.seqlens = seqlens_k;
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.H = H;
  a.Hkv = Hkv;
  a.Lmax = Lmax;
  a.d = d;
  a.c = scale * kLog2e;
  a.splits = splits;
  return FATTN_OK;
}

void set_decode_workspace(fattn::DecodeArgs& a, void* workspace) {
  a.part_o = static_cast<float*>(workspace);
  a.part_lse = a.part_o + (size_t)a.H * a.B * (a.splits + 1) * a.d;
}

}  // namespace

extern "C" {

int attn_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* seqlens_k, void* o,
                float* lse, int B, int H, int Hkv, int Lmax, int d, float scale, int num_splits, void* workspace,
                size_t workspace_bytes, void* stream) {
  const char* fn = "attn_decode";
  fattn::DecodeArgs a;
  size_t need = 0;
  bool done = false;
  const int st = prepare_decode(fn, q, k_cache, v_cache, seqlens_k, o, lse, B, H, Hkv, Lmax, d, scale, num_splits, a,
                                need, &done);
  if (st != FATTN_OK) return st;
  if (done) return ok();
  if (!workspace) return fail(FATTN_ERR_INVALID_ARG, "%s: workspace must be non-null", fn);
  if (!aligned16(workspace)) return fail(FATTN_ERR_INVALID_ARG, "%s: tensor pointers must be 16-byte aligned", fn);
  if (workspace_bytes < need)
    return fail(FATTN_ERR_INVALID_ARG, "%s: workspace of %zu bytes is smaller than the %zu required", fn,
                workspace_bytes, need);
  set_decode_workspace(a, workspace);
  return hip_status(fattn::launch_decode(a, static_cast<hipStream_t>(stream)), "attn_decode launch");
}

int attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, const int32_t* seqlens_k, void* o,
                        float* lse, int B, int H, int Hkv, int Lmax, int d, float scale, int num_splits,
                        void* stream) {
  const char* fn = "attn_decode_noalloc";
  fattn::DecodeArgs a;
  size_t need = 0;
  bool done = false;
  const int st = prepare_decode(fn, q, k_cache, v_cache, seqlens_k, o, lse, B, H, Hkv, Lmax, d, scale, num_splits, a,
                                need, &done);
  if (st != FATTN_OK) return st;
  if (done) return ok();
  if (need > fattn::kDecodeScratchBytes)
    return fail(FATTN_ERR_UNSUPPORTED, "%s: the call needs %zu bytes of workspace, more than the %zu of the static "
                "scratch array; use fewer splits or attn_decode with a workspace", fn, need,
                (size_t)fattn::kDecodeScratchBytes);
  void* scratch = nullptr;
  const hipError_t e = fattn::decode_scratch(&scratch);
  if (e != hipSuccess) return hip_status(e, "attn_decode_noalloc scratch lookup");
  set_decode_workspace(a, scratch);
  return hip_status(fattn::launch_decode(a, static_cast<hipStream_t>(stream)), "attn_decode_noalloc launch");
}

int attn_decode_paged(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                      const int32_t* seqlens_k, void* o, float* lse, int B, int H, int Hkv, int page_size,
                      int max_pages_per_seq, int num_pages, int d, float scale, int num_splits, void* workspace,
                      size_t workspace_bytes, void* stream) {
  const char* fn = "attn_decode_paged";
  if (B < 0) return fail(FATTN_ERR_INVALID_ARG, "%s: B must be >= 0 (got %d)", fn, B);
  if (H < 1 || Hkv < 1) return fail(FATTN_ERR_INVALID_ARG, "%s: H and Hkv must be >= 1", fn);
  if (H % Hkv != 0) return fail(FATTN_ERR_INVALID_ARG, "%s: H=%d is not a multiple of Hkv=%d", fn, H, Hkv);
  if (page_size < 16 || page_size > 1024 || (page_size & (page_size - 1)) != 0)
    return fail(FATTN_ERR_INVALID_ARG, "%s: page_size must be a power of two in [16, 1024] (got %d)", fn,
                page_size);
  if (max_pages_per_seq < 1 || num_pages < 1)
    return fail(FATTN_ERR_INVALID_ARG, "%s: max_pages_per_seq and num_pages must be >= 1", fn);
  if ((double)max_pages_per_seq * page_size > 2147483647.0)
    return fail(FATTN_ERR_INVALID_ARG, "%s: max_pages_per_seq*page_size too large", fn);
  if (!std::isfinite(scale) || scale < 0.f)
    return fail(FATTN_ERR_INVALID_ARG, "%s: scale must be finite and >= 0 (got %g)", fn, (double)scale);
  if (num_splits < 0 || num_splits > 64)
    return fail(FATTN_ERR_INVALID_ARG, "%s: num_splits must be 0 (auto) or 1..64 (got %d)", fn, num_splits);
  const int G = H / Hkv;
  if (d != 128) return fail(FATTN_ERR_UNSUPPORTED, "%s: d=%d not supported (128)", fn, d);
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16 && G != 32)
    return fail(FATTN_ERR_UNSUPPORTED, "%s: H/Hkv=%d not supported (1, 2, 4, 8, 16 or 32)", fn, G);
  if (B == 0) return ok();
  if (!q || !k_pages || !v_pages || !block_table || !seqlens_k || !o || !workspace)
    return fail(FATTN_ERR_INVALID_ARG, "%s: q, pages, block_table, seqlens_k, o and workspace must be non-null",
                fn);
  if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(o) || !aligned16(workspace) ||
      (lse && !aligned16(lse)))
    return fail(FATTN_ERR_INVALID_ARG, "%s: tensor pointers must be 16-byte aligned", fn);
  const int Lmax = max_pages_per_seq * page_size;
  const int splits = num_splits == 0 ? fattn::decode_auto_splits(B, Hkv, Lmax, true) : num_splits;
  // a work item holds at most ceil(ceil(Lmax / 32) / splits) blocks of 32 keys
  int chunk = (Lmax + splits - 1) / splits;
  chunk = (chunk + 31) / 32 * 32;
  if ((chunk + page_size - 1) / page_size > fattn::kDecodeMaxSplitPages)
    return fail(FATTN_ERR_UNSUPPORTED,
                "%s: one work item could span %d pages (at most %d); use more splits or larger pages",
                fn, (chunk + page_size - 1) / page_size, fattn::kDecodeMaxSplitPages);
  const size_t need = attn_decode_workspace_bytes(B, H, d, splits);
  if (workspace_bytes < need)
    return fail(FATTN_ERR_INVALID_ARG, "%s: workspace of %zu bytes is smaller than the %zu required", fn,
                workspace_bytes, need);
  int shift = 0;
  while ((1 << shift) < page_size) ++shift;
  fattn::DecodeArgs a{};
  a.q = q;
  a.k = k_pages;
  a.v = v_pages;
  a.seqlens = seqlens_k;
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.H = H;
  a.Hkv = Hkv;
  a.Lmax = Lmax;
  a.d = d;
  a.c = scale * kLog2e;
  a.splits = splits;
  a.part_o = static_cast<float*>(workspace);
  a.part_lse = a.part_o + (size_t)H * B * (splits + 1) * d;
  a.block_table = block_table;
  a.max_pages = max_pages_per_seq;
  a.page_shift = shift;
  a.num_pages = num_pages;
  return hip_status(fattn::launch_decode(a, static_cast<hipStream_t>(stream)), "attn_decode_paged launch");
}

// two f32 arrays over the query rows, each rounded up to 256 bytes: the row
// sums delta, then -LSE log2(e)
static size_t bwd_row_array_bytes(int B, int H, int N) {
  const size_t bytes = (size_t)B * H * N * sizeof(float);
  return (bytes + 255) / 256 * 256;
}

size_t attn_bwd_workspace_bytes(int B, int H, int N) {
  if (B < 0 || H < 1 || N < 0) return 0;
  return 2 * bwd_row_array_bytes(B, H, N);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
             void* dq, void* dk, void* dv, int B, int H, int Hkv, int N, int d, float scale, int causal,
             void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "attn_bwd";
  int st = check_dense(fn, q, k, v, o, lse, B, H, Hkv, N, scale, causal);
  if (st != FATTN_OK) return st;
  if (d != 64 && d != 128) return fail(FATTN_ERR_UNSUPPORTED, "%s: d=%d not supported (64 or 128)", fn, d);
  if (B == 0 || N == 0) return ok();
  if (!lse || !dout || !dq || !dk || !dv || !workspace)
    return fail(FATTN_ERR_INVALID_ARG, "%s: lse, dout, dq, dk, dv and workspace must be non-null", fn);
  if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(workspace))
    return fail(FATTN_ERR_INVALID_ARG, "%s: tensor pointers must be 16-byte aligned", fn);
  // rows of one head are addressed with 32-bit byte offsets
  if ((double)N * d * 2 >= 4294967296.0) return fail(FATTN_ERR_INVALID_ARG, "%s: N*d too large for one head", fn);
  const size_t need = attn_bwd_workspace_bytes(B, H, N);
  if (workspace_bytes < need)
    return fail(FATTN_ERR_INVALID_ARG, "%s: workspace of %zu bytes is smaller than the %zu required", fn,
                workspace_bytes, need);
  fattn::BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.delta = static_cast<float*>(workspace);
  a.nlse = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + bwd_row_array_bytes(B, H, N));
  a.B = B;
  a.H = H;
  a.Hkv = Hkv;
  a.N = N;
  a.d = d;
  a.scale = scale;
  a.c = std::fmax(scale * kLog2e, FLT_MIN);
  a.causal = causal;
  return hip_status(fattn::launch_bwd_bf16(a, static_cast<hipStream_t>(stream)), "attn_bwd launch");
}

int attn_hstu_jagged(const void* q, const void* k, const void* v, void* o, const int32_t* offsets, int B, int H,
                     int d, int max_seqlen, float alpha, float inv_n, int causal, void* stream) {
  const char* fn = "attn_hstu_jagged";
  if (B < 0 || max_seqlen < 0)
    return fail(FATTN_ERR_INVALID_ARG, "%s: B and max_seqlen must be >= 0 (got B=%d max_seqlen=%d)", fn, B,
                max_seqlen);
  if (H < 1) return fail(FATTN_ERR_INVALID_ARG, "%s: H must be >= 1", fn);
  if (causal != 0 && causal != 1) return fail(FATTN_ERR_INVALID_ARG, "%s: causal must be 0 or 1", fn);
  if (!std::isfinite(alpha) || !std::isfinite(inv_n))
    return fail(FATTN_ERR_INVALID_ARG, "%s: alpha and inv_n must be finite", fn);
  if (d != 64 && d != 128) return fail(FATTN_ERR_UNSUPPORTED, "%s: d=%d not supported (64 or 128)", fn, d);
  if (B == 0 || max_seqlen == 0) return ok();
  if (!q || !k || !v || !o || !offsets)
    return fail(FATTN_ERR_INVALID_ARG, "%s: q, k, v, o and offsets must be non-null", fn);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(FATTN_ERR_INVALID_ARG, "%s: tensor pointers must be 16-byte aligned", fn);
  // rows of one sequence are addressed with 32-bit byte offsets
  if ((double)max_seqlen * H * d * 2 >= 4294967296.0)
    return fail(FATTN_ERR_INVALID_ARG, "%s: max_seqlen*H*d too large", fn);
  fattn::TileArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = nullptr;
  a.offsets = offsets;
  a.B = B;
  a.H = H;
  a.Hkv = H;
  a.N = max_seqlen;
  a.d = d;
  a.c = alpha;
  a.inv_n = inv_n;
  a.causal = causal;
  a.epi = fattn::Epilogue::Silu;
  return hip_status(fattn::launch_tile_bf16(a, static_cast<hipStream_t>(stream)), "attn_hstu_jagged launch");
}

}  // extern "C"
