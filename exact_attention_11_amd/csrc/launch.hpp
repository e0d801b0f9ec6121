// Internal kernel launchers of libfattn (host side).  The C ABI in api.cpp
// validates arguments and then calls exactly one of these.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fattn {

// Pointwise step applied to each score of the fused tile loop.
enum class Epilogue : int {
  Softmax = 0,  // online softmax: running max, running sum, rescale
  Silu = 1,     // HSTU: silu(alpha * s), no normalisation
};

struct TileArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;              // softmax only; may be null
  const int32_t* offsets;  // jagged layout only (null for dense)
  int B, H, Hkv;
  int N;                   // dense: sequence length; jagged: max_seqlen
  int d;
  float c;                 // softmax: scale * log2(e); silu: alpha
  float inv_n;             // silu: 1/n
  int causal;
  Epilogue epi;
};

// bf16 MFMA tile kernel (dense softmax prefill or jagged SiLU).
hipError_t launch_tile_bf16(const TileArgs& a, hipStream_t stream);

struct F32Args {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  int B, H, Hkv, N, d;
  float c;  // scale * log2(e)
  int causal;
};

hipError_t launch_prefill_f32(const F32Args& a, hipStream_t stream);

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* seqlens;
  void* o;
  float* lse;
  int B, H, Hkv, Lmax, d;
  float c;  // scale * log2(e)
  int splits;       // work items per kv head: B * splits
  float* part_o;    // [H, B * (splits + 1), d]: partial of (sequence b, item w) at slot w + b
  float* part_lse;  // [H, B * (splits + 1)]
  // paged cache (block_table != null): k, v are [num_pages, Hkv, 2^page_shift, d]
  // and sequence b's logical page p is physical page block_table[b*max_pages + p]
  const int32_t* block_table;
  int max_pages;
  int page_shift;
  int num_pages;
};

// Most page-table entries one decode segment stages in LDS (a segment covers
// at most this many pages plus one).
constexpr int kDecodeMaxSplitPages = 2047;

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

// Automatic split count for a decode shape (contiguous or paged cache).
int decode_auto_splits(int B, int Hkv, int Lmax, bool paged);

// Size of the static decode scratch array (one per device, for callers that
// cannot allocate a workspace).
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;

// Device address of the current device's decode scratch array, looked up
// (hipGetSymbolAddress) on the first call on each device and kept.
hipError_t decode_scratch(void** ptr);

struct Fp8Args {
  const void* q;            // [B, H, N, d] E4M3
  const void* k;            // [B, Hkv, N, d] E4M3
  const void* v;
  void* o;                  // [B, H, N, d] bf16
  float* lse;               // [B, H, N] or null
  const float* descale_q;   // [B, H]: real value = fp8 * descale
  const float* descale_k;   // [B, Hkv]
  const float* descale_v;   // [B, Hkv]
  int B, H, Hkv, N, d;
  float c;                  // scale * log2(e)
  int causal;
};

// FP8 (E4M3) prefill tile kernel.
hipError_t launch_tile_fp8(const Fp8Args& a, hipStream_t stream);

struct BwdArgs {
  const void* q;      // [B, H, N, d] bf16
  const void* k;      // [B, Hkv, N, d] bf16
  const void* v;
  const void* o;      // forward output [B, H, N, d] bf16
  const float* lse;   // forward LSE [B, H, N] (natural log)
  const void* dout;   // dO [B, H, N, d] bf16
  void* dq;           // [B, H, N, d] bf16
  void* dk;           // [B, Hkv, N, d] bf16
  void* dv;
  float* delta;       // workspace [B, H, N]: rowsum(dO * O)
  float* nlse;        // workspace [B, H, N]: -LSE log2(e), the base-2 offset of P's exponent
  int B, H, Hkv, N, d;
  float scale;        // softmax scale
  float c;            // scale * log2(e), clamped to >= FLT_MIN
  int causal;
};

// Attention backward: dQ (and the row sums delta) by query blocks, then dK, dV
// by key blocks.
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream);

}  // namespace fattn
