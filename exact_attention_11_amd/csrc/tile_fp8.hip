// Fused exact attention with FP8 (OCP E4M3) Q, K, V on gfx950 matrix cores.
//
// The FlashAttention (TH) page's FlashAttention-3 section names FP8 support as
// one of its two hardware levers; it gives no scaling convention, so this
// kernel takes the common one: every (batch, head) slice of Q, K and V carries
// one f32 descale, the real value being fp8 * descale.  Both products run in
// FP8 with f32 accumulation (v_mfma_scale_f32_32x32x64_f8f6f4 with unit block
// scales):
//
//   S^T = K Q^T       keys on the M side, 64 d values per product;
//   O^T += V^T P^T    P rounded to E4M3 (the running-max reference keeps every
//                     weight <= 2^8, inside E4M3's range), V^T gathered from
//                     LDS by 8-bit transposing reads (ds_read_b64_tr_b8).
//
// The softmax is the bf16 kernel's (base 2, lazy rescale, in-kernel causal
// mask with tile skipping); descale_q * descale_k folds into the exponent's
// FMA and descale_v into the final 1/l.  One workgroup of four waves owns 128
// query rows of one (batch, head), 32 per wave; K and V tiles of 64 keys are
// staged through double-buffered LDS by direct HBM->LDS buffer loads (rows
// past the sequence end read as zero).  At most 168 registers per lane, so three
// workgroups (12 waves) share a CU.
//
// Lane layouts of the 32x32x64 FP8 product (A, B: lane l holds row / column
// l % 32 and k = 32 (l / 32) .. +32, one byte each; C as the 32x32 bf16
// product) make each lane's 32 P bytes of a 64-key tile the keys
// 32 (l / 32) .. +32 when the K rows are stored in LDS in the order kidx()
// below, so P^T never leaves registers.
#include <cfloat>

#include "common.hpp"
#include "launch.hpp"

namespace fattn {
namespace {

constexpr int kThreads = 256;
constexpr int kBM = 128;  // query rows per workgroup (32 per wave)
constexpr int kBN = 64;   // keys per tile
constexpr float kRescaleSlack = 8.0f;  // log2 units
constexpr int kUnitScale = 0x7f7f7f7f;  // E8M0 block scales of 1.0

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// Key (within the 64-key tile) stored in LDS row m = 32 kb + mm: accumulator
// row mm of lane half g2 = (mm >> 2) & 1 then holds key 32 g2 + 16 kb + e with
// e = 4 (mm >> 3) + (mm & 3) its element index.
__device__ __forceinline__ int kidx(int m) {
  const int kb = m >> 5, mm = m & 31;
  return 32 * ((mm >> 2) & 1) + 16 * kb + 4 * (mm >> 3) + (mm & 3);
}
// XOR on the 16-byte chunk index of a 128-byte K row: the 16 consecutive rows
// of one operand read fall on distinct banks.
__device__ __forceinline__ int swz_k(int r) { return (r >> 1) & 7; }
// Same for V rows under the 8-bit transposing read (8 consecutive rows).
__device__ __forceinline__ int swz_v(int r) { return (r >> 1) & 3; }

__device__ __forceinline__ i32x8 cat(u32x4 lo, u32x4 hi) {
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 3) void tile_fp8_kernel(Fp8Args a, int nq) {
  static_assert(D == 128, "d = 128");
  constexpr int ROW = D;                    // bytes per row
  constexpr int NKC = D / 64;               // 64-wide k-steps over d
  constexpr int NDB = D / 32;               // 32-row blocks of d in O^T
  constexpr int TILE = kBN * ROW;           // bytes of a K or V tile
  constexpr int STAGE = 2 * TILE;
  constexpr int KCH = ROW / 16;             // 16-byte chunks per row
  constexpr int NLD = kBN * KCH / kThreads; // chunks per thread per tensor
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform over the wave
  const int n32 = lane & 31;
  const int g2 = lane >> 5;

  // (batch, head, query block): a head's blocks on one XCD, heads taken four
  // at a time, heaviest blocks of a group first (measured ~2.7 % faster than
  // one head at a time)
  int slot, bh;
  grouped_item(a.B * a.H, nq, 4, bh, slot);
  const int qb = nq - 1 - slot;
  const int h = bh % a.H;
  const int b = bh / a.H;
  const int g = h / (a.H / a.Hkv);
  const int N = a.N;
  const unsigned char* qp = (const unsigned char*)a.q + ((long)b * a.H + h) * N * D;
  const unsigned char* kp = (const unsigned char*)a.k + ((long)b * a.Hkv + g) * N * D;
  const unsigned char* vp = (const unsigned char*)a.v + ((long)b * a.Hkv + g) * N * D;
  uint16_t* op = (uint16_t*)a.o + ((long)b * a.H + h) * N * D;
  // exponent scale with the descales folded in; kept >= FLT_MIN so that masked
  // scores (-inf) still give exactly 0 (as the bf16 kernel's scale = 0 case)
  const float cexp = fmaxf(a.c * a.descale_q[b * a.H + h] * a.descale_k[b * a.Hkv + g], FLT_MIN);
  const float dsv = a.descale_v[b * a.Hkv + g];

  const int q0 = qb * kBM;
  if (q0 >= N) return;
  const int kv_end = CAUSAL ? min(N, q0 + kBM) : N;
  const int n_tiles = (kv_end + kBN - 1) / kBN;
  const int q0w = q0 + 32 * wv;
  const bool wave_live = q0w < N;
  const int qrow = q0w + n32;

  // Q^T fragments (B operand): column n32 = row qrow, d = 64c + 32 g2 .. +32
  i32x8 qf[NKC];
#pragma unroll
  for (int c = 0; c < NKC; ++c) {
    u32x4 lo = {0u, 0u, 0u, 0u}, hi = lo;
    if (qrow < N) {
      lo = ldg16(qp + (long)qrow * D + 64 * c + 32 * g2);
      hi = ldg16(qp + (long)qrow * D + 64 * c + 32 * g2 + 16);
    }
    qf[c] = cat(lo, hi);
  }

  // direct HBM -> LDS tile loads: wave instruction i fills bytes (wv + 4i) KB
  // .. +1 KB of each tensor's tile.  LDS row r of K holds key kidx(r), of V
  // key r; the chunk swizzles are applied through the source address (rows
  // past the sequence end read as zero)
  constexpr int NLW = TILE / 1024 / 4;  // 1 KB loads per wave and tensor
  static_assert(NLW * 4 * 1024 == TILE, "tile split over four waves");
  uint32_t kgo[NLW], vgo[NLW];
#pragma unroll
  for (int i = 0; i < NLW; ++i) {
    const int byte = (wv + 4 * i) * 1024 + 16 * lane;
    const int r = byte / ROW, pc = (byte % ROW) / 16;
    kgo[i] = (uint32_t)kidx(r) * ROW + (uint32_t)((pc ^ swz_k(r)) << 4);
    vgo[i] = (uint32_t)r * ROW + (uint32_t)((pc ^ swz_v(r)) << 4);
  }
  const uint32_t lds0 = lds_addr_of(smem);
  auto dma_tile = [&](int k0, int buf) {
    const uint32_t bytes = (uint32_t)(N - k0) * ROW;  // rows k0 .. N-1
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kp + (long)k0 * ROW, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vp + (long)k0 * ROW, bytes);
    const uint32_t st = lds0 + (uint32_t)buf * STAGE;
#pragma unroll
    for (int i = 0; i < NLW; ++i) lds_dma16(rk, st + (wv + 4 * i) * 1024, kgo[i]);
#pragma unroll
    for (int i = 0; i < NLW; ++i) lds_dma16(rv, st + TILE + (wv + 4 * i) * 1024, vgo[i]);
  };

  // 8-bit transposing reads of V^T: within 16-lane group g4, lane j addresses
  // row 32 (g4 >> 1) + 8u + (j >> 1), bytes 32 db + 16 (g4 & 1) + 8 (j & 1)
  const int g4 = lane >> 4;
  const int j16 = lane & 15;
  const int tr_row0 = 32 * (g4 >> 1) + (j16 >> 1);
  const int tr_byte = 8 * (j16 & 1);

  f32x16 acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;
  float m_ref = kNegInf;
  float l_part = 0.f;

  dma_tile(0, 0);
  wait_vmem();
  __syncthreads();

  // Per-lane LDS byte offsets of the operand reads within a stage.  The
  // swizzles depend only on row bits the lane fixes (bits 1..3 of the key
  // row, bits 1..2 of the V row), so the 32-key block and the 8-row step of a
  // transposing read are immediate offsets: K fragment halves (c, kb) at
  // klo_off[c] / khi_off[c] + 32 kb ROW, V^T piece (db, u) at
  // v_off[db] + 8 u ROW + TILE.  With the stage a compile-time constant
  // (tiles two at a time, the inner loop unrolled) a tile adds nothing per
  // read; the empty asm keeps each offset in a register of its own.
  uint32_t klo_off[NKC], khi_off[NKC], v_off[NDB];
#pragma unroll
  for (int c = 0; c < NKC; ++c) {
    const int ch = 4 * c + 2 * g2;
    klo_off[c] = (uint32_t)(n32 * ROW + ((ch ^ swz_k(n32)) << 4));
    khi_off[c] = (uint32_t)(n32 * ROW + (((ch + 1) ^ swz_k(n32)) << 4));
    asm volatile("" : "+v"(klo_off[c]), "+v"(khi_off[c]));
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int ch = 2 * db + (g4 & 1);
    v_off[db] = (uint32_t)(tr_row0 * ROW + ((ch ^ swz_v(tr_row0)) << 4) + tr_byte);
    asm volatile("" : "+v"(v_off[db]));
  }

  for (int j0 = 0; j0 < n_tiles; j0 += 2)
#pragma unroll
  for (int su = 0; su < 2; ++su) {
    const int j = j0 + su;
    if (j >= n_tiles) break;  // uniform over the workgroup
    const int buf = su;
    const int k0 = j * kBN;
    const bool has_next = j + 1 < n_tiles;
    // the other buffer's tile was last read before the previous barrier
    if (has_next) dma_tile(k0 + kBN, buf ^ 1);

    const bool active = wave_live && !(CAUSAL && k0 > q0w + 31);
    if (active) {
      const unsigned char* sk = smem + buf * STAGE;
      const unsigned char* sv = sk + TILE;
      __builtin_amdgcn_s_setprio(1);  // products first: other waves fill the gaps with softmax work
      // S^T = K Q^T: 32-key block kb = LDS rows 32 kb .. +32
      f32x16 s[2];
      // step t = (c, kb) with kb minor: consecutive products are independent;
      // each K fragment read KW products ahead, the order pinned (reads, then
      // one product and one fragment at a time)
      constexpr int ST = 2 * NKC;
      constexpr int KW = 2;
      u32x4 klo[ST], khi[ST];
      auto kread = [&](int t) {
        const int kb = t % 2, c = t / 2;
        klo[t] = *reinterpret_cast<const u32x4*>(sk + 32 * kb * ROW + klo_off[c]);
        khi[t] = *reinterpret_cast<const u32x4*>(sk + 32 * kb * ROW + khi_off[c]);
      };
#pragma unroll
      for (int t = 0; t < KW; ++t) kread(t);
#pragma unroll
      for (int t = 0; t < ST; ++t) {
        const int kb = t % 2, c = t / 2;
        const f32x16 zero = {};
        s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cat(klo[t], khi[t]), qf[c], c == 0 ? zero : s[kb], 0,
                                                                0, 0, kUnitScale, 0, kUnitScale);
        if (t + KW < ST) kread(t + KW);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * KW, 0);
#pragma unroll
      for (int t = 0; t < ST; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (t + KW < ST) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }

      __builtin_amdgcn_s_setprio(0);
      // element e of block kb of this lane is key k0 + 32 g2 + 16 kb + e
      if ((CAUSAL && k0 + kBN - 1 > q0w) || (k0 + kBN > N)) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = k0 + 32 * g2 + 16 * kb + e;
            if (!(key < N && (!CAUSAL || key <= qrow))) s[kb][e] = kNegInf;
          }
      }
      float mt = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mt = fmaxf(mt, s[kb][e]);
      mt = max_xor32(mt);
      const float mts = mt * cexp;
      if (wave_any(mts > m_ref + kRescaleSlack)) {
        const float mn = fmaxf(m_ref, mts);
        const float alpha = (mn == kNegInf) ? 1.f : exp2_hw(m_ref - mn);
        m_ref = mn;
        l_part *= alpha;
#pragma unroll
        for (int i = 0; i < NDB; ++i)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[i][e] *= alpha;
      }
      // P^T as E4M3 bytes: byte 16 kb + e of the lane = key 32 g2 + 16 kb + e
      const float nm = -m_ref;
      i32x8 pb;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          float p[4];
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            p[x] = exp2_hw(__builtin_fmaf(s[kb][4 * w + x], cexp, nm));
            l_part += p[x];
          }
          int d = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
          d = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], d, true);
          pb[4 * kb + w] = d;
        }
      __builtin_amdgcn_s_setprio(1);
      // O^T += V^T P^T
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        i32x8 vt;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(sv + 8 * u * ROW + v_off[db]));
          vt[2 * u] = x[0];
          vt[2 * u + 1] = x[1];
        }
        acc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vt, pb, acc[db], 0, 0, 0, kUnitScale, 0,
                                                                  kUnitScale);
      }
    }

    __builtin_amdgcn_s_setprio(0);
    wait_vmem();  // this wave's pieces of the next tile have landed
    __syncthreads();
  }

  if (!wave_live || qrow >= N) return;
  const float lt = sum_xor32(l_part);
  const float scale_out = lt > 0.f ? dsv / lt : 0.f;
  if (a.lse != nullptr && g2 == 0) {
    a.lse[((long)b * a.H + h) * N + qrow] = lt > 0.f ? (m_ref + log2_hw(lt)) * kLn2 : kNegInf;
  }
  uint16_t* orow = op + (long)qrow * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int jq = 0; jq < 4; ++jq) {
      u32x2 t;
      t[0] = pack_bf16x2(acc[db][4 * jq] * scale_out, acc[db][4 * jq + 1] * scale_out);
      t[1] = pack_bf16x2(acc[db][4 * jq + 2] * scale_out, acc[db][4 * jq + 3] * scale_out);
      stg8(orow + 32 * db + 8 * jq + 4 * g2, t);
    }
}

template <int D, bool CAUSAL>
hipError_t launch_fp8_one(const Fp8Args& a, hipStream_t stream) {
  const int nq = (a.N + kBM - 1) / kBM;
  const long grid = (long)nq * a.H * a.B;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((tile_fp8_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a, nq);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tile_fp8(const Fp8Args& a, hipStream_t stream) {
  if (a.d == 128) return a.causal ? launch_fp8_one<128, true>(a, stream) : launch_fp8_one<128, false>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace fattn
