// Split-KV decode attention with a log-sum-exp combine.
//
// Decode reads every cached key and value once per step and does O(n d) work,
// so it is bound by HBM bandwidth, not by the matrix units (ledger page,
// bandwidth section).  The design therefore only tries to keep many bytes in
// flight and to touch each byte once:
//
//  * kernel 1, one 64-wide wave per (kv-head, work item): the cache rows of
//    all sequences are cut into equal runs of whole 32-key blocks, one per
//    work item, whatever the lengths (the partition below), so every wave
//    streams the same bytes and the waves finish together.  A run that crosses
//    the end of a sequence is processed as one segment per sequence.  The G
//    query heads that share the kv-head (grouped-query attention) are served
//    by the same pass, so K and V are streamed once per kv-head.  The G heads are the columns of small
//    matrix-core products (16x16x32 bf16): scores S^T = K Q^T and output
//    O^T += V^T P^T, with V^T gathered from LDS by transposing reads.  The
//    matrix cores are mostly idle doing this, but they take the dot products
//    off the vector ALUs so that the wave spends its time waiting on HBM, not
//    computing.  Online softmax per head (base 2, rescaled only when a score
//    exceeds the reference max by more than 2^8).  The next block's loads are
//    issued as soon as the current block's registers are consumed.  Each
//    segment's normalised partial output and its natural-log LSE go to the
//    workspace.
//  * kernel 2, one workgroup per (sequence, head): weights exp(lse_c - lse)
//    with lse = log-sum-exp over the sequence's partials, O = sum_c w_c o_c;
//    an empty sequence gives O = 0 and LSE = -inf.
#include <atomic>
#include <mutex>

#include "common.hpp"
#include "launch.hpp"

namespace fattn {
namespace {

// Cache rows are read once per step: stream them (cache-policy bits sc0 | nt,
// so they neither wait in L1 nor displace reusable lines in L2).  Measured on
// the GQA decode workload: ~1.8 % faster than default-policy loads.
__device__ __forceinline__ u32x4 buf_load16_stream(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 3));
}

constexpr int kD = 128;
constexpr float kRescaleSlack = 8.0f;  // log2 units
constexpr int kCombineWaves = 4;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

typedef float f32x4v __attribute__((ext_vector_type(4)));

// XOR on the 16-byte chunk index of V row r in LDS: the 8 rows one
// transposing read touches (4 per 16-lane group, two groups per LDS cycle)
// land on disjoint banks; bit 0 is never flipped, so 32-byte pieces stay whole.
__device__ __forceinline__ int v_swz(int r) { return ((r & 3) << 2) | (((r >> 2) & 1) << 1); }

// 32-key blocks of sequence b (none past the batch); L = its length clamped
// to [0, Lmax].
__device__ __forceinline__ int seq_blocks(const DecodeArgs& a, int b, int& L) {
  L = 0;
  if (b < a.B) {
    const int x = a.seqlens[b];
    L = x < 0 ? 0 : (x > a.Lmax ? a.Lmax : x);
  }
  return (L + 31) >> 5;
}

__device__ __forceinline__ long long wave_sum_ll(long long x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Work partition, shared by the split and combine kernels.  Per kv head the
// 32-key blocks of all sequences are laid end to end: sequence b holds blocks
// [P_b, P_b + nb_b), nb_b = ceil(L_b / 32), T = sum of nb_b.  With W = B *
// splits work items and W' = min(W, T), item w takes blocks
// [floor(w T / W'), floor((w + 1) T / W')): every item streams the same number
// of cache rows to within one block, whatever the lengths, so the waves finish
// together.  T >= W' makes every range non-empty, so the items touching
// sequence b are exactly those from the one holding its first block to the
// one holding its last; block x lies in item floor(((x + 1) W' - 1) / T).  An
// item crossing sequence ends writes one partial per sequence; the partial of
// (sequence b, item w) goes to slot w + b of its head.  In cache order each
// next segment raises w or b or both, so slots are distinct and below
// B * (splits + 1).
__device__ __forceinline__ long long partition_slots(const DecodeArgs& a) { return (long long)a.B * (a.splits + 1); }

// Rows [kb0, kb1) of sequence b, kv head g, by one 64-wide wave.  Blocks of
// 32 keys:
//   S^T[32 keys x 16 cols] = K Q^T   (v_mfma_f32_16x16x32_bf16, 2 x 4 steps;
//                                      column n < G is query head h0 + n, the
//                                      other columns multiply zeros)
//   online softmax per column on the accumulator (8 scores per lane)
//   O^T[128 d x 16 cols] += V^T P^T   (8 steps; V^T from LDS by transposing
//                                      reads, P^T straight from the scores)
// The normalised partial and its natural-log LSE go to slot `slot`.
template <int G, bool PAGED>
__device__ __forceinline__ void decode_segment(const DecodeArgs& a, unsigned char* sv, int* pt, int g, int b,
                                               int kb0, int kb1, long long slot) {
  constexpr int NT = G > 16 ? G / 16 : 1;  // 16-column tiles of query heads
  const int lane = threadIdx.x;
  const int n16 = lane & 15;  // column (query head) of the 16x16 tiles
  const int g4 = lane >> 4;   // 16-lane group
  const int h0 = g * G;
  const long long NS = partition_slots(a);
  float* po = a.part_o + ((long long)h0 * NS + slot) * kD;  // head h0 + hh at + hh*NS*kD
  float* pl = a.part_lse + (long long)h0 * NS + slot;       // head h0 + hh at + hh*NS

  // rows [kb0, kb1) of this kv-head; loads past kb1 read zero
  const long rowbase = ((long)b * a.Hkv + g) * a.Lmax + kb0;
  const uint32_t bytes = (uint32_t)(kb1 - kb0) * (kD * 2);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const uint16_t*)a.k + (PAGED ? 0 : rowbase * kD), bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((const uint16_t*)a.v + (PAGED ? 0 : rowbase * kD), bytes);
  const int n = kb1 - kb0;

  // paged cache: stage the block-table entries of pages lp0 .. (kb1-1)/P, plus
  // one (the half block just past the segment end), clamped to valid pages
  const int sh = a.page_shift;
  const int lp0 = kb0 >> sh;
  if constexpr (PAGED) {
    const int np = ((kb1 - 1) >> sh) - lp0 + 2;
    const int32_t* tb = a.block_table + (long)b * a.max_pages;
    for (int i = lane; i < np; i += 64) {
      const int lp = lp0 + i;
      int pg = lp < a.max_pages ? tb[lp] : 0;
      pg = pg < 0 ? 0 : (pg >= a.num_pages ? a.num_pages - 1 : pg);
      pt[i] = pg;
    }
  }

  // Q^T operand of column tile t: column n16 = head h0 + 16t + n16 (zero past
  // the group), d = 32c + 8*g4 .. +8
  bf16x8 qf[NT][4];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (16 * t + n16 < G) x = ldg16((const uint16_t*)a.q + ((long)b * a.H + h0 + 16 * t + n16) * kD + 32 * c + 8 * g4);
      qf[t][c] = as_bf16x8(x);
    }

  f32x4v acc[NT][8];
  float m[NT], l[NT];  // running (base-2, scaled) max of column n16 / this lane's share of its sum
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[t][i] = f32x4v{0.f, 0.f, 0.f, 0.f};
    m[t] = kNegInf;
    l[t] = 0.f;
  }
  const float c = a.c;

  // per-lane offsets: K operand rows n16 and 16 + n16 of a block, d = 32c + 8*g4;
  // V rows g4 + 4i (i = 0..7), d = 8*n16 .. +8
  const uint32_t koff = (uint32_t)n16 * (kD * 2) + 16u * g4;
  const uint32_t voff = (uint32_t)g4 * (kD * 2) + 16u * n16;
  // transposing reads: row 4*g4 + (lane&15)/4 (+16), d = 16*db + 4*(lane&3)
  const int tr_r = 4 * g4 + (n16 >> 2);

  u32x4 kr[8], vr[8];
  auto issue = [&](int blk) {
    if constexpr (PAGED) {
      // rows 0-15 and 16-31 of the block each lie within one page (pages
      // hold a power of two >= 16 keys, blocks start at multiples of 32)
      const int t = kb0 + blk;
      const int pA = __builtin_amdgcn_readfirstlane(pt[(t >> sh) - lp0]);
      const int pB = __builtin_amdgcn_readfirstlane(pt[((t + 16) >> sh) - lp0]);
      const int m = (1 << sh) - 1;
      const long rowA = (((long)pA * a.Hkv + g) << sh) + (t & m);
      const long rowB = (((long)pB * a.Hkv + g) << sh) + ((t + 16) & m);
      const uint32_t nA = (uint32_t)min(16, kb1 - t) * (kD * 2);
      const uint32_t nB = (uint32_t)max(0, min(16, kb1 - t - 16)) * (kD * 2);
      const __amdgpu_buffer_rsrc_t kA = make_rsrc((const uint16_t*)a.k + rowA * kD, nA);
      const __amdgpu_buffer_rsrc_t kB = make_rsrc((const uint16_t*)a.k + rowB * kD, nB);
      const __amdgpu_buffer_rsrc_t vA = make_rsrc((const uint16_t*)a.v + rowA * kD, nA);
      const __amdgpu_buffer_rsrc_t vB = make_rsrc((const uint16_t*)a.v + rowB * kD, nB);
#pragma unroll
      for (int c2 = 0; c2 < 4; ++c2) {
        kr[c2] = buf_load16_stream(kA, koff + 64u * c2);
        kr[4 + c2] = buf_load16_stream(kB, koff + 64u * c2);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) vr[i] = buf_load16_stream(i < 4 ? vA : vB, voff + (uint32_t)(4 * (i & 3)) * (kD * 2));
    } else {
      const uint32_t o = (uint32_t)blk * (kD * 2);
#pragma unroll
      for (int c2 = 0; c2 < 4; ++c2) {
        kr[c2] = buf_load16_stream(rk, o + koff + 64u * c2);
        kr[4 + c2] = buf_load16_stream(rk, o + 16u * (kD * 2) + koff + 64u * c2);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) vr[i] = buf_load16_stream(rv, o + voff + (uint32_t)(4 * i) * (kD * 2));
    }
  };

  issue(0);
  for (int blk = 0; blk < n; blk += 32) {
    // S^T for keys blk .. blk+15 (sa) and blk+16 .. blk+31 (sb), per column tile
    f32x4v sa[NT], sb[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      sa[t] = f32x4v{0.f, 0.f, 0.f, 0.f};
      sb[t] = sa[t];
#pragma unroll
      for (int c2 = 0; c2 < 4; ++c2) {
        sa[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[c2]), qf[t][c2], sa[t], 0, 0, 0);
        sb[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[4 + c2]), qf[t][c2], sb[t], 0, 0, 0);
      }
    }
    // V block -> LDS (natural [key][d] layout, swizzled chunks)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = g4 + 4 * i;
      *reinterpret_cast<u32x4*>(sv + r * (kD * 2) + ((n16 ^ v_swz(r)) << 4)) = vr[i];
    }
    if (blk + 32 < n) issue(blk + 32);

    bf16x8 pb[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      // scores of this lane: keys blk + 4*g4 + r (sa) and blk + 16 + 4*g4 + r (sb)
      float sc[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sc[r] = (blk + 4 * g4 + r < n) ? sa[t][r] * c : kNegInf;
        sc[4 + r] = (blk + 16 + 4 * g4 + r < n) ? sb[t][r] * c : kNegInf;
      }
      float mt =
          fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])), fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
      mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
      mt = max_xor32(mt);
      if (wave_any(mt > m[t] + kRescaleSlack)) {
        const float mn = fmaxf(m[t], mt);
        const float alpha = (mn == kNegInf) ? 1.f : exp2_hw(m[t] - mn);
        m[t] = mn;
        l[t] *= alpha;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[t][i] *= alpha;
      }
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = exp2_hw(sc[e] - m[t]);  // m is finite: every block has a valid key
        l[t] += p[e];
      }
      const u32x4 pw = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                        pack_bf16x2(p[6], p[7])};
      pb[t] = as_bf16x8(pw);
    }

    // O^T += V^T P^T: slots 0-3 = keys 4*g4 + t, slots 4-7 = keys 16 + 4*g4 + t
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const int chunk0 = 2 * db + ((lane & 3) >> 1);
      const int byte = 8 * (lane & 1);
      const int r0 = tr_r, r1 = tr_r + 16;
      const u32x2 lo = lds_read_tr16(sv + r0 * (kD * 2) + ((chunk0 ^ v_swz(r0)) << 4) + byte);
      const u32x2 hi = lds_read_tr16(sv + r1 * (kD * 2) + ((chunk0 ^ v_swz(r1)) << 4) + byte);
      const u32x4 vf = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
      for (int t = 0; t < NT; ++t)
        acc[t][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vf), pb[t], acc[t][db], 0, 0, 0);
    }
  }

  // row sum over the four 16-lane groups; normalise and write the partial
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float lt = l[t] + __shfl_xor(l[t], 16, 64);
    lt = sum_xor32(lt);
    const int hh = 16 * t + n16;  // head within the group
    if (hh < G) {
      const float inv = 1.f / lt;
      float* dst = po + (long long)hh * NS * kD + 4 * g4;
#pragma unroll
      for (int db = 0; db < 8; ++db)
        stg16(dst + 16 * db, u32x4{__float_as_uint(acc[t][db][0] * inv), __float_as_uint(acc[t][db][1] * inv),
                                   __float_as_uint(acc[t][db][2] * inv), __float_as_uint(acc[t][db][3] * inv)});
      if (g4 == 0) pl[(long long)hh * NS] = (m[t] + log2_hw(lt)) * kLn2;
    }
  }
}

// One 64-wide wave per (kv head, work item): walks the segments of its block
// range in cache order.
template <int G, bool PAGED>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char sv[32 * kD * 2];
  // paged cache: physical page of each logical page one segment touches
  __shared__ int pt[PAGED ? kDecodeMaxSplitPages + 2 : 1];
  const int lane = threadIdx.x;
  const int g = blockIdx.x % a.Hkv;
  const long long w = blockIdx.x / a.Hkv;

  long long T = 0;
  for (int base = 0; base < a.B; base += 64) {
    int L;
    T += wave_sum_ll(seq_blocks(a, base + lane, L));
  }
  const long long W = (long long)a.B * a.splits;
  const long long Wp = W < T ? W : T;
  if (w >= Wp) return;  // also every wave when all sequences are empty
  const long long lo = w * T / Wp, hi = (w + 1) * T / Wp;

  long long carry = 0;  // blocks of the sequences before this group of 64
  for (int base = 0; base < a.B && carry < hi; base += 64) {
    int L;
    const int nb = seq_blocks(a, base + lane, L);
    long long x = nb;  // inclusive prefix sum over the group
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const long long y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    const long long P = carry + x - nb;
    unsigned long long act = __ballot((P > lo ? P : lo) < (P + nb < hi ? P + nb : hi));
    while (act) {
      const int i = __builtin_ctzll(act);
      act &= act - 1;
      const long long Pb = __shfl(P, i, 64);
      const int Lb = __builtin_amdgcn_readfirstlane(__shfl(L, i, 64));
      const long long s0 = Pb > lo ? Pb : lo;
      const long long e = Pb + ((Lb + 31) >> 5);
      const long long s1 = e < hi ? e : hi;
      const int kb0 = __builtin_amdgcn_readfirstlane((int)((s0 - Pb) * 32));
      const int kb1 = __builtin_amdgcn_readfirstlane(min(Lb, (int)((s1 - Pb) * 32)));
      decode_segment<G, PAGED>(a, sv, pt, g, base + i, kb0, kb1, w + base + i);
    }
    carry += __shfl(x, 63, 64);
  }
}

// One workgroup per (sequence, head).  The partials of sequence b are the
// slots of the work items that touch it (see the partition above), found from
// the same prefix sums; wave w sums slots w, w+4, ...; every lane owns 2 d
// values.
__global__ __launch_bounds__(64 * kCombineWaves) void decode_combine_kernel(DecodeArgs a) {
  __shared__ float part[kCombineWaves][kD];
  const int bh = blockIdx.x;
  const int b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;

  long long T = 0, P = 0;
  for (int base = 0; base < a.B; base += 64) {
    int L;
    const int nb = seq_blocks(a, base + lane, L);
    T += wave_sum_ll(nb);
    P += wave_sum_ll(base + lane < b ? nb : 0);
  }
  int Lb;
  const int nbb = seq_blocks(a, b, Lb);
  uint16_t* o = (uint16_t*)a.o + (long)bh * kD;
  if (nbb == 0) {  // empty sequence (uniform over the workgroup)
    if (tid < kD / 2) reinterpret_cast<uint32_t*>(o)[tid] = 0u;
    if (a.lse != nullptr && tid == 0) a.lse[bh] = kNegInf;
    return;
  }
  const long long W = (long long)a.B * a.splits;
  const long long Wp = W < T ? W : T;
  const long long wf = ((P + 1) * Wp - 1) / T;    // item holding the first block
  const long long wl = ((P + nbb) * Wp - 1) / T;  // item holding the last block
  const int n = (int)(wl - wf + 1);
  const long long NS = partition_slots(a);
  const float* pl = a.part_lse + (long long)h * NS + wf + b;
  const float* po = a.part_o + ((long long)h * NS + wf + b) * kD;

  float M, Wsum, acc0 = 0.f, acc1 = 0.f;
  constexpr int kPerWave = 64 / kCombineWaves;
  if (n <= 64) {
    // one load of every LSE and every partial row this wave sums, all issued
    // before the reductions that weight them
    const float ls = lane < n ? pl[lane] : kNegInf;
    float2 v[kPerWave];
#pragma unroll
    for (int k = 0; k < kPerWave; ++k) {
      const int s = wv + kCombineWaves * k;
      v[k] = s < n ? *reinterpret_cast<const float2*>(po + (long)s * kD + 2 * lane) : make_float2(0.f, 0.f);
    }
    M = wave_max(ls);
    const float w = lane < n ? exp2_hw((ls - M) * kLog2e) : 0.f;
    Wsum = wave_sum(w);
#pragma unroll
    for (int k = 0; k < kPerWave; ++k) {
      const float ws = __shfl(w, wv + kCombineWaves * k, 64);
      acc0 = __builtin_fmaf(ws, v[k].x, acc0);
      acc1 = __builtin_fmaf(ws, v[k].y, acc1);
    }
  } else {
    M = kNegInf;
    for (int i = lane; i < n; i += 64) M = fmaxf(M, pl[i]);
    M = wave_max(M);
    Wsum = 0.f;
    for (int i = lane; i < n; i += 64) Wsum += exp2_hw((pl[i] - M) * kLog2e);
    Wsum = wave_sum(Wsum);
    for (int i0 = 0; i0 < n; i0 += 64) {
      const float w = i0 + lane < n ? exp2_hw((pl[i0 + lane] - M) * kLog2e) : 0.f;
      // 16 slots per wave, all loads independent
#pragma unroll
      for (int k = 0; k < kPerWave; ++k) {
        const int s = wv + kCombineWaves * k;
        const float ws = __shfl(w, s, 64);
        if (i0 + s < n) {
          const float2 v = *reinterpret_cast<const float2*>(po + (long)(i0 + s) * kD + 2 * lane);
          acc0 = __builtin_fmaf(ws, v.x, acc0);
          acc1 = __builtin_fmaf(ws, v.y, acc1);
        }
      }
    }
  }
  part[wv][2 * lane] = acc0;
  part[wv][2 * lane + 1] = acc1;
  __syncthreads();
  if (tid < kD / 2) {
    float r0 = 0.f, r1 = 0.f;
#pragma unroll
    for (int x = 0; x < kCombineWaves; ++x) {
      r0 += part[x][2 * tid];
      r1 += part[x][2 * tid + 1];
    }
    const float inv = 1.f / Wsum;
    reinterpret_cast<uint32_t*>(o)[tid] = pack_bf16x2(r0 * inv, r1 * inv);
  }
  if (a.lse != nullptr && tid == 0) a.lse[bh] = M + log2_hw(Wsum) * kLn2;
}

template <int G>
hipError_t launch_g(const DecodeArgs& a, hipStream_t stream) {
  const long grid = (long)a.Hkv * a.B * a.splits;
  if (a.block_table != nullptr) {
    hipLaunchKernelGGL((decode_split_kernel<G, true>), dim3((unsigned)grid), dim3(64), 0, stream, a);
  } else {
    hipLaunchKernelGGL((decode_split_kernel<G, false>), dim3((unsigned)grid), dim3(64), 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3((unsigned)((long)a.B * a.H)), dim3(64 * kCombineWaves), 0, stream,
                     a);
  return hipGetLastError();
}

}  // namespace

int decode_auto_splits(int B, int Hkv, int Lmax, bool paged) {
  // About 768 work items (three per CU) for a contiguous cache and 1024 for
  // a paged one, whose extra page-table step per block wants more waves in
  // flight.  The B * Hkv * splits items start together and, streaming equal
  // runs, finish together.  Measured on the GQA decode workload
  // (B * Hkv = 128), contiguous: 768 items 6.68 TB/s, 512 6.56, 1024 6.59,
  // 1536 6.54, 2048 6.37; paged (16-key pages): 768 6.00, 1024 6.40, 1536
  // 6.10, 2048 6.19.  Counts that leave the CUs unevenly loaded are slower
  // (contiguous, 896: 6.10, 2560: 5.86).  The work items a sequence of Lmax
  // keys would get hold at least 256 keys each, and at most the keys of
  // kDecodeMaxSplitPages pages of the smallest size (16 keys); at most 64
  // splits.
  const long pairs = (long)B * Hkv;
  long s = pairs > 0 ? (paged ? 1024 : 768) / pairs : 64;
  const long smax = (Lmax + 255) / 256;
  if (s > smax) s = smax;
  const long item_max = (long)kDecodeMaxSplitPages * 16 / 32 * 32;  // whole 32-key blocks
  const long smin = (Lmax + item_max - 1) / item_max;
  if (s < smin) s = smin;
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  return (int)s;
}

// Decode workspace for callers that cannot allocate (attn_decode_noalloc):
// kDecodeScratchBytes per device, held until the process ends.  In host code
// the name `scratch` stands for the array but is not its device address; the
// address is looked up once per device with that device current and only that
// address is passed to kernels.  Every call on one device shares the array:
// calls that overlap on a device race.  Its contents on entry do not matter
// (the split kernel writes every slot the combine reads), so nothing clears it.
static __device__ __attribute__((aligned(256))) unsigned char scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t decode_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.d != kD) return hipErrorInvalidValue;
  if (a.B == 0) return hipSuccess;
  switch (a.H / a.Hkv) {
    case 1: return launch_g<1>(a, stream);
    case 2: return launch_g<2>(a, stream);
    case 4: return launch_g<4>(a, stream);
    case 8: return launch_g<8>(a, stream);
    case 16: return launch_g<16>(a, stream);
    case 32: return launch_g<32>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fattn
