// Split-KV decode attention with a log-sum-exp combine, on the vector ALUs.
//
// Decode reads every cached key and value once per step and does O(n d) work,
// so it is bound by HBM bandwidth, not by the matrix units (ledger page,
// bandwidth section).  The design therefore only tries to keep enough bytes in
// flight and to touch each byte once:
//
//  * kernel 1, one workgroup per (sequence, kv-head, split): the split owns a
//    contiguous chunk of cache rows.  The G query heads that share the kv-head
//    (grouped-query attention) are served by the same pass, so K and V are
//    streamed once per kv-head.  Each 16-lane row group of a wave handles one
//    key: lane i holds 8 consecutive d values (one 16-byte load), dot products
//    use v_dot2_f32_bf16 and a 4-step DPP butterfly within the row.  Scores of
//    a sub-chunk go to LDS, then max and exponentials (base 2), then V is
//    streamed and p * v accumulated in f32.  Sub-chunks are merged online
//    (running max and sum, as in the prefill kernel).  The normalised partial
//    output and its natural-log LSE go to the workspace; an empty chunk
//    writes 0 and -inf.
//  * kernel 2, one workgroup per (sequence, head): weights exp(lse_c - lse)
//    with lse = log-sum-exp over the splits, O = sum_c w_c o_c.
#include "common.hpp"
#include "launch.hpp"

namespace fattn {
namespace {

constexpr int kD = 128;
constexpr int kSub = 512;    // keys per scored sub-chunk
constexpr int kUnroll = 8;   // 16-key steps issued back to back
constexpr int kThreads = 256;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the total.
__device__ __forceinline__ float row16_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));  // quad [1,0,3,2]
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));  // quad [2,3,0,1]
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false)); // half-row mirror
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false)); // row mirror
  return x;
}

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

template <int G>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeArgs a, int chunk) {
  __shared__ float sc[G][kSub];
  __shared__ float stat[G][2];
  __shared__ float red[4][G][kD];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int kk = 4 * wv + (lane >> 4);  // key slot within a 16-key step
  const int ds = lane & 15;             // 8-wide d slice

  const int S = a.splits;
  int wid = blockIdx.x;
  const int s = wid % S;
  wid /= S;
  const int g = wid % a.Hkv;
  const int b = wid / a.Hkv;
  const int h0 = g * G;

  int L = a.seqlens[b];
  L = L < 0 ? 0 : (L > a.Lmax ? a.Lmax : L);
  const int kb0 = s * chunk;
  const int kb1 = min(L, kb0 + chunk);

  float* po = a.part_o + (((long)b * a.H + h0) * S + s) * kD;  // head hh at + hh*S*kD
  float* pl = a.part_lse + ((long)b * a.H + h0) * S + s;       // head hh at + hh*S

  if (kb0 >= kb1) {
    for (int i = tid; i < G * kD; i += kThreads) po[(long)(i / kD) * S * kD + (i % kD)] = 0.f;
    if (tid < G) pl[(long)tid * S] = kNegInf;
    return;
  }

  const long kvbase = ((long)b * a.Hkv + g) * a.Lmax * kD;
  const uint16_t* kp = (const uint16_t*)a.k + kvbase + 8 * ds;
  const uint16_t* vp = (const uint16_t*)a.v + kvbase + 8 * ds;

  uint32_t qv[G][4];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const u32x4 t = ldg16((const uint16_t*)a.q + ((long)b * a.H + h0 + hh) * kD + 8 * ds);
    qv[hh][0] = t[0];
    qv[hh][1] = t[1];
    qv[hh][2] = t[2];
    qv[hh][3] = t[3];
  }

  float acc[G][8];
  float m_run[G], l_run[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m_run[hh] = kNegInf;
    l_run[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[hh][e] = 0.f;
  }
  const float c = a.c;

  for (int sb = kb0; sb < kb1; sb += kSub) {
    const int se = min(kb1, sb + kSub);
    const int n = se - sb;

    // pass A: scaled base-2 scores of the sub-chunk into LDS
    for (int base = sb; base < se; base += 16 * kUnroll) {
      u32x4 kv[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int key = base + 16 * u + kk;
        u32x4 t = {0u, 0u, 0u, 0u};
        if (key < se) t = ldg16(kp + (long)key * kD);
        kv[u] = t;
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int key = base + 16 * u + kk;
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          float p = dot2(qv[hh][0], kv[u][0], 0.f);
          p = dot2(qv[hh][1], kv[u][1], p);
          p = dot2(qv[hh][2], kv[u][2], p);
          p = dot2(qv[hh][3], kv[u][3], p);
          p = row16_sum(p);
          if (ds == hh && key < se) sc[hh][key - sb] = p * c;
        }
      }
    }
    __syncthreads();

    // sub-chunk max, exponentials and sum; wave wv serves heads wv, wv+4, ...
    for (int hh = wv; hh < G; hh += 4) {
      float mx = kNegInf;
      for (int i = lane; i < n; i += 64) mx = fmaxf(mx, sc[hh][i]);
      mx = wave_max(mx);
      // m_run is the same in every thread, so this wave can fix the new
      // reference max for head hh and publish it with the sum below.
      float sum = 0.f;
      const float mnew = fmaxf(m_run[hh], mx);
      for (int i = lane; i < n; i += 64) {
        const float p = exp2_hw(sc[hh][i] - mnew);
        sc[hh][i] = p;
        sum += p;
      }
      sum = wave_sum(sum);
      if (lane == 0) {
        stat[hh][0] = mnew;
        stat[hh][1] = sum;
      }
    }
    __syncthreads();

#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float mnew = stat[hh][0];
      const float alpha = (m_run[hh] == kNegInf) ? 0.f : exp2_hw(m_run[hh] - mnew);
      m_run[hh] = mnew;
      l_run[hh] = l_run[hh] * alpha + stat[hh][1];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hh][e] *= alpha;
    }

    // pass B: stream V, accumulate p * v
    for (int base = sb; base < se; base += 16 * kUnroll) {
      u32x4 vv[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int key = base + 16 * u + kk;
        u32x4 t = {0u, 0u, 0u, 0u};
        if (key < se) t = ldg16(vp + (long)key * kD);
        vv[u] = t;
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int key = base + 16 * u + kk;
        const bool in = key < se;
        float vf[8];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          vf[2 * w] = bf16_lo(vv[u][w]);
          vf[2 * w + 1] = bf16_hi(vv[u][w]);
        }
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const float p = in ? sc[hh][min(key - sb, kSub - 1)] : 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[hh][e] = __builtin_fmaf(p, vf[e], acc[hh][e]);
        }
      }
    }
    __syncthreads();  // sc and stat are rewritten by the next sub-chunk
  }

  // reduce over the 4 key slots of a wave (lanes l, l^16, l^32, l^48) ...
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = acc[hh][e];
      x += __shfl_xor(x, 16, 64);
      x += __shfl_xor(x, 32, 64);
      acc[hh][e] = x;
    }
  // ... then over the 4 waves through LDS
  if (lane < 16) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) red[wv][hh][8 * ds + e] = acc[hh][e];
  }
  __syncthreads();
  for (int i = tid; i < G * kD; i += kThreads) {
    const int hh = i / kD, dd = i % kD;
    const float sum = red[0][hh][dd] + red[1][hh][dd] + red[2][hh][dd] + red[3][hh][dd];
    float lsum = 0.f;
#pragma unroll
    for (int x = 0; x < G; ++x)
      if (x == hh) lsum = l_run[x];
    po[(long)hh * S * kD + dd] = sum / lsum;
  }
  if (tid < G) {
    float mm = 0.f, ll = 1.f;
#pragma unroll
    for (int x = 0; x < G; ++x)
      if (x == tid) {
        mm = m_run[x];
        ll = l_run[x];
      }
    pl[(long)tid * S] = (mm + log2_hw(ll)) * kLn2;
  }
}

__global__ __launch_bounds__(kD) void decode_combine_kernel(DecodeArgs a) {
  const int bh = blockIdx.x;
  const int dd = threadIdx.x;
  const int S = a.splits;
  const float* pl = a.part_lse + (long)bh * S;
  const float* po = a.part_o + (long)bh * S * kD;
  float M = kNegInf;
  for (int s = 0; s < S; ++s) M = fmaxf(M, pl[s]);
  uint16_t* o = (uint16_t*)a.o + (long)bh * kD;
  if (M == kNegInf) {
    o[dd] = 0;
    if (a.lse != nullptr && dd == 0) a.lse[bh] = kNegInf;
    return;
  }
  float wsum = 0.f, acc = 0.f;
  for (int s = 0; s < S; ++s) {
    const float w = exp2_hw((pl[s] - M) * kLog2e);
    wsum += w;
    acc = __builtin_fmaf(w, po[(long)s * kD + dd], acc);
  }
  const float r = acc / wsum;
  const uint32_t packed = pack_bf16x2(r, 0.f);
  o[dd] = (uint16_t)(packed & 0xffffu);
  if (a.lse != nullptr && dd == 0) a.lse[bh] = M + log2_hw(wsum) * kLn2;
}

template <int G>
hipError_t launch_g(const DecodeArgs& a, int chunk, hipStream_t stream) {
  const long grid = (long)a.B * a.Hkv * a.splits;
  hipLaunchKernelGGL(decode_split_kernel<G>, dim3((unsigned)grid), dim3(kThreads), 0, stream, a, chunk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3((unsigned)((long)a.B * a.H)), dim3(kD), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

int decode_auto_splits(int B, int Hkv, int Lmax) {
  // Chunks of about 512 keys, at most 64 splits.
  int s = (Lmax + 511) / 512;
  if (s < 1) s = 1;
  if (s > 64) s = 64;
  (void)B;
  (void)Hkv;
  return s;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.d != kD) return hipErrorInvalidValue;
  if (a.B == 0) return hipSuccess;
  int chunk = (a.Lmax + a.splits - 1) / a.splits;
  chunk = (chunk + 15) / 16 * 16;
  if (chunk < 16) chunk = 16;
  switch (a.H / a.Hkv) {
    case 1: return launch_g<1>(a, chunk, stream);
    case 2: return launch_g<2>(a, chunk, stream);
    case 4: return launch_g<4>(a, chunk, stream);
    case 8: return launch_g<8>(a, chunk, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fattn
