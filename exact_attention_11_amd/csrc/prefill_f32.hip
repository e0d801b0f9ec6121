// Exact attention in f32 end to end (inputs, probabilities, accumulation).
//
// A plain tiled online-softmax kernel on the vector ALUs: one 64-wide wave per
// workgroup, one query row per lane, K and V tiles of 64 keys staged in LDS and
// read as broadcasts.  Per tile every lane computes its 64 scores, updates its
// running max, rescales its output and running sum once, then accumulates
// p * v (CANN ops-transformer FlashAttention page, steps 1-4 of the solution).
// This path serves small f32 problems where exactness, not speed, matters.
#include "common.hpp"
#include "launch.hpp"

namespace fattn {
namespace {

constexpr int kD = 64;
constexpr int kBK = 64;

template <bool CAUSAL>
__global__ __launch_bounds__(64) void prefill_f32_kernel(F32Args a, int nq) {
  __shared__ float sk[kBK][kD];
  __shared__ float sv[kBK][kD];
  const int lane = threadIdx.x;
  int wid = blockIdx.x;
  const int qb = wid % nq;
  wid /= nq;
  const int h = wid % a.H;
  const int b = wid / a.H;
  const int g = h / (a.H / a.Hkv);
  const int N = a.N;
  const long qbase = ((long)b * a.H + h) * N * kD;
  const long kbase = ((long)b * a.Hkv + g) * N * kD;
  const int qrow = qb * 64 + lane;
  const bool live = qrow < N;

  float q[kD], o[kD];
#pragma unroll
  for (int c = 0; c < kD; ++c) {
    q[c] = live ? a.q[qbase + (long)qrow * kD + c] : 0.f;
    o[c] = 0.f;
  }
  float m = kNegInf, l = 0.f;
  const int kv_end = CAUSAL ? min(N, qb * 64 + 64) : N;

  for (int k0 = 0; k0 < kv_end; k0 += kBK) {
    __syncthreads();
    for (int i = lane; i < kBK * kD; i += 64) {
      const int r = i / kD, c = i % kD;
      const bool in = k0 + r < N;
      sk[r][c] = in ? a.k[kbase + (long)(k0 + r) * kD + c] : 0.f;
      sv[r][c] = in ? a.v[kbase + (long)(k0 + r) * kD + c] : 0.f;
    }
    __syncthreads();
    float s[kBK];
    float mt = kNegInf;
#pragma unroll
    for (int j = 0; j < kBK; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < kD; ++c) acc = __builtin_fmaf(q[c], sk[j][c], acc);
      const int key = k0 + j;
      const bool vis = key < N && (!CAUSAL || key <= qrow);
      s[j] = vis ? acc * a.c : kNegInf;
      mt = fmaxf(mt, s[j]);
    }
    const float mn = fmaxf(m, mt);
    if (mn == kNegInf) continue;  // nothing visible yet for this row
    const float alpha = exp2_hw(m - mn);
    m = mn;
    l *= alpha;
#pragma unroll
    for (int c = 0; c < kD; ++c) o[c] *= alpha;
#pragma unroll
    for (int j = 0; j < kBK; ++j) {
      const float p = exp2_hw(s[j] - m);
      l += p;
#pragma unroll
      for (int c = 0; c < kD; ++c) o[c] = __builtin_fmaf(p, sv[j][c], o[c]);
    }
  }
  if (!live) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int c = 0; c < kD; ++c) a.o[qbase + (long)qrow * kD + c] = o[c] * inv;
  if (a.lse != nullptr) a.lse[((long)b * a.H + h) * N + qrow] = l > 0.f ? (m + log2_hw(l)) * kLn2 : kNegInf;
}

}  // namespace

hipError_t launch_prefill_f32(const F32Args& a, hipStream_t stream) {
  if (a.d != kD) return hipErrorInvalidValue;
  const int nq = (a.N + 63) / 64;
  const long grid = (long)nq * a.H * a.B;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
  if (a.causal)
    hipLaunchKernelGGL(prefill_f32_kernel<true>, dim3((unsigned)grid), dim3(64), 0, stream, a, nq);
  else
    hipLaunchKernelGGL(prefill_f32_kernel<false>, dim3((unsigned)grid), dim3(64), 0, stream, a, nq);
  return hipGetLastError();
}

}  // namespace fattn
