// Fused, tiled exact attention on gfx950 matrix cores (bf16 in, fp32 accumulate).
//
// One workgroup of four 64-wide waves owns 128 query rows of one (batch, head);
// each wave owns 32 of them.  K and V tiles stream from HBM through LDS (double
// buffered, one barrier per tile) while the score tile and the output
// accumulator stay in registers, so the N x N score matrix never reaches HBM
// (CANN ops-transformer FlashAttention page: tiles sized to the matrix unit,
// block results kept on chip, only the final output written back).
//
// Per tile the wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (keys on
// the M side, queries on the N side).  The accumulator then holds, in each lane,
// 16 scores of ONE query column, which is (a) the layout of the B operand of the
// next product O^T += V^T P^T, so P never leaves registers, and (b) makes the
// row max and row sum mostly in-lane: only lanes l and l^32 share a query.
//
// Keys are fed to the first product in a permuted row order (bits 2 and 3 of the
// in-block key index swapped) so that each lane's 8 P values for one K=16 step
// of the second product are 8 CONSECUTIVE keys.  V stays in its natural
// [key][d] layout in LDS and the V^T operand is gathered with the transposing
// LDS read (ds_read_b64_tr_b16): two reads give a lane 8 consecutive keys of
// one d column.  V rows are XOR-swizzled in 16-byte chunks so that the four key
// rows one read touches fall in different banks.
//
// K and V tiles go straight from HBM into LDS (buffer_load ... lds: no
// staging registers, no LDS store instructions in the wave), the next tile's
// loads issued into the free buffer as a tile starts and waited for at its
// barrier.  The load descriptor covers only the valid rows of the sequence:
// rows past the end read as zero, so no load is predicated.
//
// Two pointwise epilogues share the loop:
//  * Softmax: online softmax with a running row max m and running sum l
//    (CANN ops-transformer FlashAttention page, steps 1-4; FlashAttention (TH)
//    page, online softmax).  Scores are handled in base 2 with scale*log2(e)
//    folded into one FMA.  The output is rescaled only when some row's tile max
//    exceeds the reference max by more than 2^8 -- between rescales every
//    exponent is relative to a common reference that is at most 8 below the
//    true running max, so weights stay <= 256 and the final O/l and LSE are
//    the same quantities.
//  * Silu: HSTU pointwise attention, silu(alpha s) with no normalisation
//    (HSTU page, the listing and optimisation one).  Q is multiplied by
//    alpha*log2(e) as it is loaded, so the product is t = log2(e) alpha s and
//    a weight is t / (1 + 2^-t) = log2(e) silu(alpha s); the epilogue's 1/n
//    takes the factor ln 2.  (d = 128; the d = 64 HSTU kernel at the end of
//    this file splits each query block's keys between two wave pairs.)
//
// Causal masking is generated in the kernel from tile positions: tiles wholly
// below the diagonal run unmasked, tiles straddling it are masked per element,
// tiles wholly above it are never loaded or computed (HSTU page, optimisation
// two).  Rows and keys past the sequence end (ragged N, jagged sequences) are
// masked the same way.
#include "common.hpp"
#include "launch.hpp"

namespace fattn {
namespace {

constexpr int kThreads = 256;
constexpr int kBM = 128;              // query rows per workgroup
constexpr float kRescaleSlack = 8.0f;  // log2 units

// Keys per K/V tile.  Smaller tiles leave room for more waves per SIMD: with
// 32-key tiles the d = 128 kernel needs at most 168 registers and 32 KB of LDS,
// so three workgroups (12 waves) share a CU; the d = 64 kernel fits four
// (at most 128 registers, 32 KB).  Every wave's step is a serial chain
// (products, softmax, products); more waves per SIMD keep the matrix cores fed
// while some of them are in the softmax.
template <int D>
struct Cfg;
//
// kHeadGroup: heads of an XCD whose query blocks are dispatched together
// (unpaired grids), heaviest first.  Larger groups end the launch with lighter
// blocks but keep more heads' K/V live in the XCD's 4 MB L2, so more of it is
// fetched again from HBM: measured on the causal B=8, H=32, N=4096 workload,
// groups of 4 against 2 were ~1.4 % faster for d = 128 (1.88 against 1.35 GB
// of HBM traffic per launch, 1.08 GB algorithmic) and ~4 % for d = 256; 16 and
// more were slower.
//
// kKAhead / kVAhead: LDS operand reads kept in flight ahead of the products
// (K fragments of the score product, V^T fragments of the PV product); 0
// leaves the order to the compiler.  With the three-level wave priorities of
// the tile loop, 3 and 2 measured ~1 % faster than 3 and 3, 2 and 2 or 4 and 4
// for d = 128, and ~1.5 % faster than the compiler's order for d = 64; d = 256
// (one wave per SIMD) is fastest with 3 and 3.
// Per-lane LDS offsets of a tile kernel's operand reads; empty where the
// kernel computes its addresses in the loop.
template <bool ON, int NK, int NV>
struct LaneOffsets {
  uint32_t ka[NK], va[NV];
};
template <int NK, int NV>
struct LaneOffsets<false, NK, NV> {
  uint32_t* ka = nullptr;
  uint32_t* va = nullptr;
};

template <>
struct Cfg<128> {
  static constexpr int BN = 32;
  static constexpr int kWavesPerSimd = 3;
  static constexpr int kHeadGroup = 4;
  static constexpr int kKAhead = 3;
  static constexpr int kVAhead = 2;
  static constexpr bool kStagePairs = true;
};
template <>
struct Cfg<256> {
  // the d = 256 output accumulator (128 registers per lane) and Q fragments
  // (64) leave no room for more; one workgroup per CU, one wave per SIMD,
  // accumulators in the AGPR half of the register file
  static constexpr int BN = 32;
  static constexpr int kWavesPerSimd = 1;
  static constexpr int kHeadGroup = 4;
  static constexpr int kKAhead = 3;
  static constexpr int kVAhead = 3;
  static constexpr bool kStagePairs = true;
};
template <>
struct Cfg<64> {
  static constexpr int BN = 64;
  static constexpr int kWavesPerSimd = 4;
  static constexpr int kHeadGroup = 2;
  static constexpr int kKAhead = 3;
  static constexpr int kVAhead = 2;
  static constexpr bool kStagePairs = false;
};

// Layout of one K/V stage filled by direct HBM->LDS loads (1 KB of
// consecutive LDS bytes per wave instruction, so no row padding): rows of D
// bf16 whose 16-byte chunks are XOR-swizzled, by kswz for K and vswz for V.
template <int D, int BN>
struct Lds {
  static constexpr int kRow = D * 2;
  static constexpr int kBytes = BN * kRow;
  static constexpr int vRow = D * 2;
  static constexpr int vBytes = BN * vRow;
  static constexpr int stage = kBytes + vBytes;
  static constexpr int total = 2 * stage;
  // 16 lanes of a K fragment read (16 distinct rows, one chunk column) hit 16
  // distinct 16-byte bank groups
  __device__ static __forceinline__ int kswz(int r) { return D == 64 ? ((r >> 1) & 7) : (r & 15); }
  // the 4 consecutive rows a transposing read touches land on disjoint banks
  // (bits >= 2 of the chunk index only, so 32-byte pieces stay contiguous)
  __device__ static __forceinline__ int vswz(int r) { return D >= 128 ? ((r & 3) << 2) : ((r & 2) << 1); }
};

// Rows [s0, s1) of packed sequence b: offsets[b] and offsets[b + 1] clamped
// into [0, offsets[B]] with s1 >= s0, so that offsets that are out of order or
// out of range never address a row outside [0, offsets[B]).
__device__ __forceinline__ void jagged_rows(const TileArgs& a, int b, int& s0, int& s1) {
  const int total = max(a.offsets[a.B], 0);
  s0 = min(max(a.offsets[b], 0), total);
  s1 = min(max(a.offsets[b + 1], s0), total);
}

// In-block key order of the first product: swap bits 2 and 3.
__device__ __forceinline__ int key_perm(int m) { return (m & ~0xC) | ((m & 4) << 1) | ((m & 8) >> 1); }

// Key (relative to the 32-key block) held by accumulator element e = 4j + r of
// a lane in half g2 (lane / 32).
__device__ __forceinline__ int acc_key(int e, int g2) {
  const int j = e >> 2, r = e & 3;
  return 16 * (j >> 1) + 8 * g2 + 4 * (j & 1) + r;
}

template <int D, bool CAUSAL, Epilogue EPI, bool JAGGED>
__global__ __launch_bounds__(kThreads, Cfg<D>::kWavesPerSimd) void tile_kernel(TileArgs a, int nq, int pair) {
  constexpr int BN = Cfg<D>::BN;
  constexpr int NKB = BN / 32;  // 32-key blocks per tile
  constexpr int NDB = D / 32;   // 32-row blocks of d
  constexpr int NDC = D / 16;   // K=16 steps over d
  using L = Lds<D, BN>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[L::total];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform over the wave
  const int n32 = lane & 31;
  const int g2 = lane >> 5;

  // ---- work item: (batch, head, slot), all slots of a head on one XCD.
  // Unpaired: slot = one query block; each XCD takes its heads kHeadGroup at
  // a time, heaviest query blocks of a group first (one head at a time left a
  // ~10 % tail of heavy blocks started late).  Paired (causal grids that fit
  // on the chip at once): slot i runs query blocks nqb-1-i and i, so every
  // workgroup does the same work and no CU is left with the heaviest blocks.
  const int nslot = pair ? (nq + 1) / 2 : nq;
  int slot, bh;
  grouped_item(a.B * a.H, nslot, pair ? 1 : Cfg<D>::kHeadGroup, bh, slot);
  const int h = bh % a.H;
  const int b = bh / a.H;

  const uint16_t* qp;
  const uint16_t* kp;
  const uint16_t* vp;
  uint16_t* op;
  long row_stride;  // elements between consecutive rows
  int len;
  long lse_base = 0;
  if constexpr (JAGGED) {
    int s0, s1;
    jagged_rows(a, b, s0, s1);
    len = min(s1 - s0, a.N);
    row_stride = (long)a.H * D;
    const long base = ((long)s0 * a.H + h) * D;
    qp = (const uint16_t*)a.q + base;
    kp = (const uint16_t*)a.k + base;
    vp = (const uint16_t*)a.v + base;
    op = (uint16_t*)a.o + base;
  } else {
    len = a.N;
    row_stride = D;
    const int g = h / (a.H / a.Hkv);
    const long qbase = ((long)b * a.H + h) * a.N * D;
    const long kbase = ((long)b * a.Hkv + g) * a.N * D;
    qp = (const uint16_t*)a.q + qbase;
    op = (uint16_t*)a.o + qbase;
    kp = (const uint16_t*)a.k + kbase;
    vp = (const uint16_t*)a.v + kbase;
    lse_base = ((long)b * a.H + h) * a.N;
  }
  auto run_block = [&](const int qb) {
    const int q0 = qb * kBM;
    if (len <= 0 || q0 >= len) return;  // uniform over the workgroup

    const int kv_end = CAUSAL ? min(len, q0 + kBM) : len;
    const int n_tiles = (kv_end + BN - 1) / BN;

    const int q0w = q0 + 32 * wv;
    const bool wave_live = q0w < len;
    const int qrow = q0w + n32;

    // ---- Q fragments (B operand of S^T = K Q^T), kept in registers.
    bf16x8 qf[NDC];
#pragma unroll
    for (int c = 0; c < NDC; ++c) {
      u32x4 t = {0u, 0u, 0u, 0u};
      if (qrow < len) t = ldg16(qp + (long)qrow * row_stride + 16 * c + 8 * g2);
      if constexpr (EPI == Epilogue::Silu) {
        // HSTU: Q scaled by log2(e) alpha (rounded to bf16), so the product is
        // the exponent t of the SiLU weight directly
        const float beta = a.c * kLog2e;
#pragma unroll
        for (int x = 0; x < 4; ++x) t[x] = pack_bf16x2(bf16_lo(t[x]) * beta, bf16_hi(t[x]) * beta);
      }
      qf[c] = as_bf16x8(t);
    }

    // ---- direct HBM -> LDS loads of one K/V tile: wave instruction i fills
    // bytes (wv + 4i) KB .. +1 KB of each tensor's tile; the chunk swizzles are
    // applied through the source address (rows past the sequence end read as
    // zero)
    constexpr int NLW = BN * D * 2 / 1024 / 4;  // 1 KB loads per wave and tensor
    static_assert(NLW * 4 * 1024 == BN * D * 2, "tile split over four waves");
    const uint32_t row_bytes = (uint32_t)row_stride * 2;
    uint32_t koff[NLW], voff[NLW];
#pragma unroll
    for (int i = 0; i < NLW; ++i) {
      const int byte = (wv + 4 * i) * 1024 + 16 * lane;
      const int r = byte / (D * 2);
      const int pc = (byte % (D * 2)) / 16;
      koff[i] = (uint32_t)r * row_bytes + (uint32_t)(pc ^ L::kswz(r)) * 16u;
      voff[i] = (uint32_t)r * row_bytes + (uint32_t)(pc ^ L::vswz(r)) * 16u;
    }
    const uint32_t lds0 = lds_addr_of(smem);
    auto dma_tile = [&](int k0, int buf) {
      const uint32_t bytes = (uint32_t)(len - k0 - 1) * row_bytes + D * 2;
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(kp + (long)k0 * row_stride, bytes);
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(vp + (long)k0 * row_stride, bytes);
      const uint32_t st = lds0 + (uint32_t)buf * L::stage;
#pragma unroll
      for (int i = 0; i < NLW; ++i) lds_dma16(rk, st + (wv + 4 * i) * 1024, koff[i]);
#pragma unroll
      for (int i = 0; i < NLW; ++i) lds_dma16(rv, st + L::kBytes + (wv + 4 * i) * 1024, voff[i]);
    };

    // per-lane part of the transposing V^T reads: row offset within the 8-key
    // group and (chunk, byte) of the 4 d values this lane addresses
    const int tr_row = (lane & 15) >> 2;
    const int tr_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    const int tr_byte = 8 * (lane & 1);

    // Per-lane LDS byte offsets of the operand reads within a stage.  The
    // swizzles depend only on the low row bits a lane fixes (kswz on bits
    // 0..3 of the key row, vswz on bits 0..1 of the V row), so the 32-key
    // block, the 16-row half and the upper 4 rows of a transposing read are
    // immediate offsets: K fragment (c, kb) is at ka[c] + 32 kb kRow, V^T
    // fragment (kb, jj, db) at va[db] + (32 kb + 16 jj) vRow.  The empty asm
    // keeps each offset in a register of its own, so the tile loop adds
    // nothing per read.
    LaneOffsets<Cfg<D>::kStagePairs, NDC, NDB> lo;
    uint32_t* const ka = lo.ka;
    uint32_t* const va = lo.va;
    if constexpr (Cfg<D>::kStagePairs) {
      const int kr0 = key_perm(n32);
#pragma unroll
      for (int c = 0; c < NDC; ++c) {
        ka[c] = (uint32_t)(kr0 * L::kRow + (((2 * c + g2) ^ L::kswz(kr0)) << 4));
        asm volatile("" : "+v"(ka[c]));
      }
      const int vr0 = 8 * g2 + tr_row;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        va[db] = (uint32_t)(vr0 * L::vRow + (((4 * db + tr_chunk) ^ L::vswz(vr0)) << 4) + tr_byte);
        asm volatile("" : "+v"(va[db]));
      }
    }

    // ---- accumulators and running statistics
    f32x16 acc[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;
    float m_ref = kNegInf;  // base-2 reference max (scaled)
    float l_part = 0.f;     // this lane's share of the row sum
    const float cexp = a.c;

    dma_tile(0, 0);
    wait_vmem();
    __syncthreads();

    // Tiles go two at a time where the stage pairs are on: the inner loop is
    // unrolled, so the LDS stage is a compile-time constant and every LDS
    // read of a tile is one per-lane address register plus an immediate
    // offset, with no address arithmetic per read.
    constexpr int SU = Cfg<D>::kStagePairs ? 2 : 1;
    for (int j0 = 0; j0 < n_tiles; j0 += SU)
#pragma unroll
    for (int su = 0; su < SU; ++su) {
      const int j = j0 + su;
      if (SU > 1 && j >= n_tiles) break;  // uniform over the workgroup
      const int buf = SU > 1 ? su : (j & 1);
      const int k0 = j * BN;
      const bool has_next = j + 1 < n_tiles;
      // the other buffer's tile was last read before the previous barrier
      if (has_next) dma_tile(k0 + BN, buf ^ 1);

      const bool active = wave_live && !(CAUSAL && k0 > q0w + 31);
      if (active) {
        const unsigned char* sk = smem + buf * L::stage;
        const unsigned char* sv = sk + L::kBytes;
        // Wave priorities: output products 2, score products 1, softmax 0.
        // Products go first, so other waves fill the matrix cores' gaps with
        // their softmax work; among products, a wave finishing its tile goes
        // before one starting a tile (both at one level measured ~3 % slower).
        __builtin_amdgcn_s_setprio(1);
        // S^T = K Q^T
        f32x16 s[NKB];
        auto kread = [&](int c, int kb) {
          if constexpr (Cfg<D>::kStagePairs) return *reinterpret_cast<const u32x4*>(sk + 32 * kb * L::kRow + ka[c]);
          const int kr_ = 32 * kb + key_perm(n32);
          return *reinterpret_cast<const u32x4*>(sk + kr_ * L::kRow + (((2 * c + g2) ^ L::kswz(kr_)) << 4));
        };
        if constexpr (Cfg<D>::kKAhead == 0) {
#pragma unroll
          for (int c = 0; c < NDC; ++c)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
              const f32x16 zero = {};
              s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kread(c, kb)), qf[c], c == 0 ? zero : s[kb], 0,
                                                              0, 0);
            }
        } else {
          // each K fragment read KW products ahead of its use; the schedule is
          // pinned: KW reads, then one product and one read at a time
          constexpr int SSTEPS = NDC * NKB;
          constexpr int KW = Cfg<D>::kKAhead < SSTEPS ? Cfg<D>::kKAhead : SSTEPS;
          u32x4 kf[SSTEPS];
#pragma unroll
          for (int t = 0; t < KW; ++t) kf[t] = kread(t / NKB, t % NKB);
#pragma unroll
          for (int t = 0; t < SSTEPS; ++t) {
            const int c = t / NKB, kb = t % NKB;
            const f32x16 zero = {};
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf[t]), qf[c], c == 0 ? zero : s[kb], 0, 0, 0);
            if (t + KW < SSTEPS) kf[t + KW] = kread((t + KW) / NKB, (t + KW) % NKB);
          }
          __builtin_amdgcn_sched_group_barrier(0x100, KW, 0);  // DS reads
#pragma unroll
          for (int t = 0; t < SSTEPS; ++t) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            if (t + KW < SSTEPS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
        }

        __builtin_amdgcn_s_setprio(0);
        const bool masked = (CAUSAL && k0 + BN - 1 > q0w) || (k0 + BN > len);
        // visibility of accumulator element e of 32-key block kb
        auto visible = [&](int kb, int e) {
          const int key = k0 + 32 * kb + acc_key(e, g2);
          return (key < len) && (!CAUSAL || key <= qrow);
        };

        uint32_t pk[NKB][8];  // bf16 pairs of P (or of silu scores)
        if constexpr (EPI == Epilogue::Softmax) {
          // Masked scores become -inf; with cexp > 0 (the host never passes 0)
          // their weights exp2(-inf) are exactly 0, with no per-element select.
          if (masked) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
              for (int e = 0; e < 16; ++e)
                if (!visible(kb, e)) s[kb][e] = kNegInf;
          }
          float mt = kNegInf;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) mt = fmaxf(mt, s[kb][e]);
          mt = max_xor32(mt);
          const float mts = mt * cexp;  // -inf stays -inf
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
          const float nm = -m_ref;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
            float p[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              p[e] = exp2_hw(__builtin_fmaf(s[kb][e], cexp, nm));
              l_part += p[e];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) pk[kb][e] = pack_bf16x2(p[2 * e], p[2 * e + 1]);
          }
        } else {
          // the product is t = log2(e) alpha s (Q carries the factor):
          // t / (1 + 2^-t) = log2(e) silu(alpha s); the factor log2(e) comes off
          // in the epilogue's scale
          float y[NKB][16];
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const float t = s[kb][e];
              y[kb][e] = t * rcp_hw(1.f + exp2_hw(-t));
            }
          if (masked) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
              for (int e = 0; e < 16; ++e)
                if (!visible(kb, e)) y[kb][e] = 0.f;
          }
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int e = 0; e < 8; ++e) pk[kb][e] = pack_bf16x2(y[kb][2 * e], y[kb][2 * e + 1]);
        }

        __builtin_amdgcn_s_setprio(2);
        // O^T += V^T P^T; V^T fragments gathered by transposing reads
        auto vread = [&](int kb, int jj, int db) {
          const int krow = 32 * kb + 16 * jj + 8 * g2 + tr_row;
          const unsigned char* addr =
              Cfg<D>::kStagePairs ? sv + (32 * kb + 16 * jj) * L::vRow + va[db]
                                  : sv + krow * L::vRow + (((4 * db + tr_chunk) ^ L::vswz(krow)) << 4) + tr_byte;
          const u32x2 lo = lds_read_tr16(addr);
          const u32x2 hi = lds_read_tr16(addr + 4 * L::vRow);
          return u32x4{lo[0], lo[1], hi[0], hi[1]};
        };
        auto pfrag = [&](int kb, int jj) {
          const u32x4 pw = {pk[kb][4 * jj], pk[kb][4 * jj + 1], pk[kb][4 * jj + 2], pk[kb][4 * jj + 3]};
          return as_bf16x8(pw);
        };
        if constexpr (Cfg<D>::kVAhead == 0) {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
              for (int db = 0; db < NDB; ++db)
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vread(kb, jj, db)), pfrag(kb, jj), acc[db],
                                                                  0, 0, 0);
        } else {
          // each V^T fragment read PW products ahead of its use (pinned as above)
          constexpr int PSTEPS = NKB * 2 * NDB;
          constexpr int PW = Cfg<D>::kVAhead < PSTEPS ? Cfg<D>::kVAhead : PSTEPS;
          u32x4 vfr[PSTEPS];
          auto vstep = [&](int t) { return vread(t / (2 * NDB), (t / NDB) % 2, t % NDB); };
#pragma unroll
          for (int t = 0; t < PW; ++t) vfr[t] = vstep(t);
#pragma unroll
          for (int t = 0; t < PSTEPS; ++t) {
            const int kb = t / (2 * NDB), jj = (t / NDB) % 2, db = t % NDB;
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vfr[t]), pfrag(kb, jj), acc[db], 0, 0, 0);
            if (t + PW < PSTEPS) vfr[t + PW] = vstep(t + PW);
          }
          __builtin_amdgcn_sched_group_barrier(0x100, 2 * PW, 1);
#pragma unroll
          for (int t = 0; t < PSTEPS; ++t) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
            if (t + PW < PSTEPS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
          }
        }
      }

      __builtin_amdgcn_s_setprio(0);
      wait_vmem();      // this wave's pieces of the next tile have landed
      __syncthreads();  // everyone's have; this tile's buffer is free
    }

    if (!wave_live || qrow >= len) return;

    float scale_out;
    if constexpr (EPI == Epilogue::Softmax) {
      const float lt = sum_xor32(l_part);
      scale_out = lt > 0.f ? 1.f / lt : 0.f;
      if (a.lse != nullptr && g2 == 0) {
        a.lse[lse_base + qrow] = lt > 0.f ? (m_ref + log2_hw(lt)) * kLn2 : kNegInf;
      }
    } else {
      scale_out = a.inv_n * kLn2;  // the weights carry a factor log2(e)
    }
    uint16_t* orow = op + (long)qrow * row_stride;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        u32x2 t;
        t[0] = pack_bf16x2(acc[db][4 * jq] * scale_out, acc[db][4 * jq + 1] * scale_out);
        t[1] = pack_bf16x2(acc[db][4 * jq + 2] * scale_out, acc[db][4 * jq + 3] * scale_out);
        stg8(orow + 32 * db + 8 * jq + 4 * g2, t);
      }
  };

  if (!pair) {
    run_block(nq - 1 - slot);
  } else {
    const int nqb = (min(len, a.N) + kBM - 1) / kBM;  // query blocks of this sequence
    const int j = nqb - 1 - slot;
    if (slot > j) return;  // uniform over the workgroup
    run_block(j);
    if (j != slot) run_block(slot);  // the previous block ended with a barrier: LDS is free
  }
}

template <int D, bool CAUSAL, Epilogue EPI, bool JAGGED>
hipError_t launch_one(const TileArgs& a, hipStream_t stream) {
  const int nq = (a.N + kBM - 1) / kBM;
  // causal work per query block grows with its index; when the paired grid
  // fits on the chip at once (256 CUs x resident workgroups), balance it
  const long resident = 256L * Cfg<D>::kWavesPerSimd;
  const int pair = (CAUSAL && (long)((nq + 1) / 2) * a.H * a.B <= resident) ? 1 : 0;
  const long grid = (long)(pair ? (nq + 1) / 2 : nq) * a.H * a.B;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((tile_kernel<D, CAUSAL, EPI, JAGGED>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a, nq,
                     pair);
  return hipGetLastError();
}

template <int D, Epilogue EPI, bool JAGGED>
hipError_t launch_causal(const TileArgs& a, hipStream_t s) {
  return a.causal ? launch_one<D, true, EPI, JAGGED>(a, s) : launch_one<D, false, EPI, JAGGED>(a, s);
}

// ---------------------------------------------------------------------------
// Jagged HSTU, d = 64: the key tiles of each query block are split between two
// pairs of waves.  A workgroup owns 64 query rows; wave w takes rows
// 32 (w & 1) .. +32 and the key tiles of parity w >> 1, so the longest chain of
// a launch (the last query block of the longest sequence) walks half the keys
// it would with one wave per row group.  The two partial sums of a row group
// (plain sums: the SiLU weights are not normalised) meet in LDS in a fixed
// order at the end, so results do not depend on timing; with the tiles split
// by parity, zero-padded keys past a sequence only add exact zeros to either
// sum, so a zero-padded batch gives the jagged result bit for bit.
// Work item of a jagged launch balanced over the 8 XCDs (blockIdx % 8 is the
// XCD a workgroup is dispatched to).  The (sequence, head) pairs are ranked by
// sequence length, longest first (ties by index), and dealt to the XCDs in
// snake order -- ranks 0..7 to XCDs 0..7, ranks 8..15 to XCDs 7..0, and so
// on -- so every XCD gets a near-equal share of the quadratic work while all
// query blocks of a pair stay on one XCD (its K and V in that XCD's L2).  Each
// XCD's workgroups take its existing query blocks in a dense list, heaviest
// first, and the workgroups past the list (the grid covers every pair at the
// longest length) return false at the end of it.  The hardware starts the
// workgroups in block order, each on its XCD, waiting while that XCD is full:
// with the blocks past a short sequence's end spread through the order, the
// XCDs holding the long sequences filled up early and held back the others
// (2.5 workgroups per CU resident on the jagged workload, against 4 for
// equal lengths).  One lane per sequence ranks the lengths (B <= 64) and one
// lane per pair of the XCD counts its blocks (B*H <= 512).  Also returns the
// sequence's first row and length.
__device__ __forceinline__ bool balanced_jagged_item(const TileArgs& a, int& b, int& h, int& qb, int& s0b, int& lenb) {
  const int lane = threadIdx.x & 63;
  int len = -1;  // lanes past the batch rank after every sequence
  int s0 = 0;
  if (lane < a.B) {
    int s1;
    jagged_rows(a, lane, s0, s1);
    len = min(s1 - s0, a.N);
  }
  int rank = 0;  // sequences before this one: longer, or as long with a smaller index
  for (int t = 0; t < a.B; ++t) {
    const int lt = __builtin_amdgcn_readlane(len, t);
    rank += (lt > len || (lt == len && t < lane)) ? 1 : 0;
  }
  // lane r: length of the sequence of rank r
  const int len_by_rank = __builtin_amdgcn_ds_permute(4 * (lane < a.B ? rank : lane), len);
  const int npairs = a.B * a.H;
  const int x = blockIdx.x & 7;
  const int u = blockIdx.x >> 3;
  // lane k: this XCD's pair k, sorted pair i = 8 k + (k even ? x : 7 - x),
  // with nb_k = ceil(L / 64) query blocks (non-increasing in k).  The XCD's
  // items are listed densely, heaviest first: query block qb descending, then
  // pair k, only blocks that exist (blocks nb_{k+1} .. nb_k - 1 exist for
  // pairs 0 .. k); workgroups past the list have no item.
  // (the shuffles run in every lane: a lane reads only active lanes)
  const int ik = 8 * lane + ((lane & 1) ? 7 - x : x);
  const int lk = __shfl(len_by_rank, min(ik / a.H, 63));
  const int nb = ik < npairs ? (lk + 63) >> 6 : 0;
  const int nb_up = __shfl(nb, (lane + 1) & 63);
  const int nbn = lane < 63 ? nb_up : 0;
  const int cnt = (nb - nbn) * (lane + 1);
  int pre = cnt;  // inclusive prefix sum over the lanes
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(pre, o);
    if (lane >= o) pre += t;
  }
  const unsigned long long found = __ballot(pre > u);
  if (found == 0) return false;
  const int k = __builtin_ctzll(found);
  const int v = u - __builtin_amdgcn_readlane(pre - cnt, k);
  const int q = v / (k + 1), j = v - q * (k + 1);
  qb = __builtin_amdgcn_readlane(nb, k) - 1 - q;
  const int ij = 8 * j + ((j & 1) ? 7 - x : x);
  const int sr = ij / a.H;
  h = ij - sr * a.H;
  b = __builtin_ctzll(__ballot(lane < a.B && rank == sr));
  s0b = __builtin_amdgcn_readlane(s0, b);
  lenb = __builtin_amdgcn_readlane(len, b);
  return true;
}

template <bool CAUSAL>
__global__ __launch_bounds__(kThreads, 4) void hstu_split_kernel(TileArgs a, int nqb, int balanced) {
  constexpr int D = 64;
  constexpr int BN = 32;
  constexpr int BMW = 64;      // query rows per workgroup
  constexpr int NDB = D / 32;  // 32-row blocks of d
  constexpr int NDC = D / 16;  // K=16 steps over d
  using L = Lds<D, BN>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[4 * L::stage];  // 2 key halves x 2 stages
  static_assert(4 * L::stage >= 2 * NDB * 16 * 64 * 4 * 2, "room for the partial sums");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wv & 1;   // row group
  const int ks = wv >> 1;  // key half
  const int n32 = lane & 31;
  const int g2 = lane >> 5;

  int b, h, qb, s0, len;
  if (balanced) {
    if (!balanced_jagged_item(a, b, h, qb, s0, len)) return;  // uniform over the workgroup
  } else {
    int slot, bh;
    grouped_item(a.B * a.H, nqb, 4, bh, slot);
    h = bh % a.H;
    b = bh / a.H;
    qb = nqb - 1 - slot;  // heaviest blocks first
    int s1;
    jagged_rows(a, b, s0, s1);
    len = min(s1 - s0, a.N);
  }
  const int q0 = qb * BMW;
  if (q0 >= len) return;  // uniform over the workgroup
  const long rs = (long)a.H * D;           // elements between consecutive rows
  const long base = ((long)s0 * a.H + h) * D;
  const uint16_t* qp = (const uint16_t*)a.q + base;
  const uint16_t* kp = (const uint16_t*)a.k + base;
  const uint16_t* vp = (const uint16_t*)a.v + base;
  uint16_t* op = (uint16_t*)a.o + base;

  const int kv_end = CAUSAL ? min(len, q0 + BMW) : len;
  const int n_tiles = (kv_end + BN - 1) / BN;
  const int steps = (n_tiles + 1) / 2;  // step t: tile 2t (even half) and 2t+1 (odd half)
  const int q0w = q0 + 32 * rg;
  const bool wave_live = q0w < len;
  const int qrow = q0w + n32;

  // step t loads tiles 2t and 2t+1 straight into LDS: wave instruction w
  // fills bytes w KB .. +1 KB of each tensor's tile (the chunk swizzles applied
  // through the source address)
  const uint32_t row_bytes = (uint32_t)rs * 2;
  static_assert(BN * D * 2 == 4 * 1024, "one 1 KB load per wave, tile and tensor");
  uint32_t koff, voff;
  {
    const int byte = wv * 1024 + 16 * lane;
    const int r = byte / (D * 2), pc = (byte % (D * 2)) / 16;
    koff = (uint32_t)r * row_bytes + (uint32_t)((pc ^ L::kswz(r)) << 4);
    voff = (uint32_t)r * row_bytes + (uint32_t)((pc ^ L::vswz(r)) << 4);
  }
  // one descriptor per tensor over rows [0, len) of this head: rows past the
  // sequence end read as zero
  const uint32_t seq_bytes = (uint32_t)(len - 1) * row_bytes + D * 2;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kp, seq_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vp, seq_bytes);
  const uint32_t lds0 = lds_addr_of(smem);
  // A tile past the key range (the odd half of the last step) is not loaded:
  // the waves of that half skip the step.
  auto dma_step = [&](int t, int buf) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int ti = 2 * t + st;
      if (ti < n_tiles) {
        const uint32_t off = (uint32_t)ti * (BN * row_bytes);
        const uint32_t sk = lds0 + (uint32_t)(st * 2 + buf) * L::stage;
        lds_dma16(rk, sk + wv * 1024, off + koff);
        lds_dma16(rv, sk + L::kBytes + wv * 1024, off + voff);
      }
    }
  };

  const int tr_row = (lane & 15) >> 2;
  const int tr_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int tr_byte = 8 * (lane & 1);

  f32x16 acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;

  dma_step(0, 0);  // in flight while the Q fragments load
  // Q fragments, scaled by alpha log2(e) as in the tile kernel
  bf16x8 qf[NDC];
  const float beta = a.c * kLog2e;
#pragma unroll
  for (int c = 0; c < NDC; ++c) {
    u32x4 t = {0u, 0u, 0u, 0u};
    if (qrow < len) t = ldg16(qp + (long)qrow * rs + 16 * c + 8 * g2);
#pragma unroll
    for (int x = 0; x < 4; ++x) t[x] = pack_bf16x2(bf16_lo(t[x]) * beta, bf16_hi(t[x]) * beta);
    qf[c] = as_bf16x8(t);
  }

  wait_vmem();
  __syncthreads();
  // Per-lane LDS byte offsets of the operand reads (this wave's key half
  // included); the swizzles depend only on low row bits the lane fixes, so
  // the 16-row half and the upper 4 rows of a transposing read are immediate
  // offsets, and with the stage a compile-time constant (steps taken two at
  // a time) the step adds nothing per read.
  uint32_t ka[NDC], va[NDB];
  {
    const int kr0 = key_perm(n32);
    const int vr0 = 8 * g2 + tr_row;
#pragma unroll
    for (int c = 0; c < NDC; ++c) {
      ka[c] = (uint32_t)(ks * 2 * L::stage + kr0 * L::kRow + (((2 * c + g2) ^ L::kswz(kr0)) << 4));
      asm volatile("" : "+v"(ka[c]));
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      va[db] = (uint32_t)(ks * 2 * L::stage + L::kBytes + vr0 * L::vRow +
                          (((4 * db + tr_chunk) ^ L::vswz(vr0)) << 4) + tr_byte);
      asm volatile("" : "+v"(va[db]));
    }
  }

  for (int t0 = 0; t0 < steps; t0 += 2)
#pragma unroll
  for (int su = 0; su < 2; ++su) {
    const int t = t0 + su;
    if (t >= steps) break;  // uniform over the workgroup
    const int buf = su;
    const bool has_next = t + 1 < steps;
    // the other buffers' tiles were last read before the previous barrier
    if (has_next) dma_step(t + 1, buf ^ 1);
    const int ti = 2 * t + ks;
    const int k0 = ti * BN;
    const bool active = wave_live && ti < n_tiles && !(CAUSAL && k0 > q0w + 31);
    if (active) {
      const unsigned char* sb = smem + buf * L::stage;
      __builtin_amdgcn_s_setprio(1);
      f32x16 s;
#pragma unroll
      for (int c = 0; c < NDC; ++c) {
        const u32x4 kf = *reinterpret_cast<const u32x4*>(sb + ka[c]);
        const f32x16 zero = {};
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf), qf[c], c == 0 ? zero : s, 0, 0, 0);
      }
      __builtin_amdgcn_s_setprio(0);
      // t / (1 + 2^-t) = log2(e) silu(alpha s); masked keys weigh 0
      float y[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) y[e] = s[e] * rcp_hw(1.f + exp2_hw(-s[e]));
      if ((CAUSAL && k0 + BN - 1 > q0w) || (k0 + BN > len)) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = k0 + acc_key(e, g2);
          if (!((key < len) && (!CAUSAL || key <= qrow))) y[e] = 0.f;
        }
      }
      uint32_t pk[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pk[e] = pack_bf16x2(y[2 * e], y[2 * e + 1]);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const u32x4 pw = {pk[4 * jj], pk[4 * jj + 1], pk[4 * jj + 2], pk[4 * jj + 3]};
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const unsigned char* addr = sb + 16 * jj * L::vRow + va[db];
          const u32x2 lo = lds_read_tr16(addr);
          const u32x2 hi = lds_read_tr16(addr + 4 * L::vRow);
          const u32x4 vf = {lo[0], lo[1], hi[0], hi[1]};
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf), as_bf16x8(pw), acc[db], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
    wait_vmem();  // this wave's pieces of the next step's tiles have landed
    __syncthreads();
  }

  // the odd-tile waves hand their partial sums to the even-tile waves (same
  // lane layout)
  float* red = reinterpret_cast<float*>(smem) + rg * (NDB * 16 * 64);
  if (ks == 1) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) red[(db * 16 + e) * 64 + lane] = acc[db][e];
  }
  __syncthreads();
  if (ks == 1 || !wave_live || qrow >= len) return;
  const float scale_out = a.inv_n * kLn2;  // the weights carry a factor log2(e)
  uint16_t* orow = op + (long)qrow * rs;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int jq = 0; jq < 4; ++jq) {
      float v4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v4[r] = (acc[db][4 * jq + r] + red[(db * 16 + 4 * jq + r) * 64 + lane]) * scale_out;
      u32x2 t;
      t[0] = pack_bf16x2(v4[0], v4[1]);
      t[1] = pack_bf16x2(v4[2], v4[3]);
      stg8(orow + 32 * db + 8 * jq + 4 * g2, t);
    }
}

template <bool CAUSAL>
hipError_t launch_hstu_split(const TileArgs& a, hipStream_t stream) {
  const int nqb = (a.N + 63) / 64;
  // XCD-balanced order when one wave can rank the sequences and count one XCD's
  // pairs, and there are enough (sequence, head) pairs for every XCD
  const long npairs = (long)a.H * a.B;
  const int balanced = (a.B <= 64 && npairs >= 8 && npairs <= 512) ? 1 : 0;
  const long grid = balanced ? 8L * ((npairs + 7) / 8) * nqb : (long)nqb * npairs;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((hstu_split_kernel<CAUSAL>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a, nqb,
                     balanced);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tile_bf16(const TileArgs& a, hipStream_t stream) {
  if (a.epi == Epilogue::Softmax) {
    if (a.d == 128) return launch_causal<128, Epilogue::Softmax, false>(a, stream);
    if (a.d == 64) return launch_causal<64, Epilogue::Softmax, false>(a, stream);
    if (a.d == 256) return launch_causal<256, Epilogue::Softmax, false>(a, stream);
  } else {
    if (a.d == 128) return launch_causal<128, Epilogue::Silu, true>(a, stream);
    if (a.d == 64) return a.causal ? launch_hstu_split<true>(a, stream) : launch_hstu_split<false>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace fattn
