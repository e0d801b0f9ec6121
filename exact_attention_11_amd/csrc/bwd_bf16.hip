// Attention backward on gfx950 matrix cores (bf16 in, fp32 accumulate).
//
// Given Q, K, V, the forward output O and its LSE, and dO, the gradients are
// those of O = softmax(scale Q K^T) V (the chain rule of the forward
// definition; the ledger page's memory section names the backward pass and
// its n x n intermediates, which are never materialised here):
//
//   P = exp(scale Q K^T - LSE)      recomputed from the saved LSE
//   dV = P^T dO,  dP = dO V^T,  delta_i = sum_c dO_ic O_ic
//   dS = P * (dP - delta),  dQ = scale dS K,  dK = scale dS^T Q
//
// Two kernels, neither uses atomics:
//  * bwd_dq_kernel, one workgroup per 128 query rows of a (batch, head), in
//    the forward kernel's layout: per key tile S^T = K Q^T and dP^T = V dO^T
//    (32x32x16 products, keys on the M side), dS^T in registers, then
//    dQ^T += K^T dS^T with K^T gathered by transposing LDS reads.  It also
//    computes delta for its rows (from dO and O, already in registers for the
//    fragment loads) and stores it, with -LSE log2(e) of each row, for the
//    second kernel.
//  * bwd_dkdv_kernel, one workgroup of 8 waves per 128 keys of a (batch,
//    kv-head): four wave pairs of 32 keys each, the keys being the columns of
//    32x32x16 products.  Per tile of 64 query rows (of every query head of
//    the group) the first wave of a pair computes S = Q K^T, P, and
//    dV^T += dO^T P; the second, one tile behind, dP = dO V^T, dS with the P
//    its partner left in LDS, and dK^T += Q^T dS; dO^T and Q^T come from
//    transposing reads.  Splitting the products over the pair keeps each
//    wave's registers (one K or V operand, one accumulator) within the half of
//    the register file that two waves per SIMD allow, while 32 keys per wave
//    halve the LDS bytes per product against 16.  The group's query heads
//    accumulate in registers.
// K/V tiles (first kernel) stream into LDS double buffered, Q/dO tiles
// (second kernel) into a ring of three, with direct HBM->LDS loads and one
// barrier per tile.  Causal tiles wholly above the diagonal are skipped,
// straddling tiles masked per element.
#include <cfloat>

#include "common.hpp"
#include "launch.hpp"

namespace fattn {
namespace {

constexpr int kThreads = 256;
constexpr int kBM = 128;  // query rows per dQ workgroup (32 per wave)
constexpr int kBN = 64;   // keys per dQ tile
constexpr int kBQ = 64;   // query rows per step of the dK/dV loop
constexpr int kKB = 128;  // keys per dK/dV workgroup (32 per wave pair)
constexpr int kPairThreads = 512;

// XOR on the 16-byte chunk index of row r of a K or V tile (dQ kernel) or a Q
// or dO tile (dK/dV kernel).  The plain operand reads (16 lanes, 16
// consecutive rows, one logical chunk) and the transposing reads (4
// consecutive rows, 32 bytes each) both fall on distinct banks.
template <int D>
__device__ __forceinline__ int swz_kv(int r) {
  return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}
// In-block row order of the first products (keys in the dQ kernel, queries in
// the dK/dV kernel): swap bits 2, 3.
__device__ __forceinline__ int key_perm(int m) { return (m & ~0xC) | ((m & 4) << 1) | ((m & 8) >> 1); }

// Key (relative to the 32-key block) held by accumulator element e = 4j + r of
// a lane in half g2 (lane / 32).
__device__ __forceinline__ int acc_key(int e, int g2) {
  const int j = e >> 2, r = e & 3;
  return 16 * (j >> 1) + 8 * g2 + 4 * (j & 1) + r;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(BwdArgs a, int nq) {
  constexpr int NKB = kBN / 32;
  constexpr int NDB = D / 32;
  constexpr int NDC = D / 16;
  constexpr int ROW = D * 2;            // bytes per row
  constexpr int TILE = kBN * ROW;       // bytes of a K or V tile
  constexpr int NLD = TILE / 1024 / 4;  // 1 KB direct loads per wave per tile
  static_assert(TILE % 4096 == 0, "tile split over four waves");
  __shared__ __attribute__((aligned(16))) unsigned char smem[4 * TILE];  // 2 stages x (K, V)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n32 = lane & 31;
  const int g2 = lane >> 5;

  // (batch, head, query block): all blocks of a head on one XCD, heads taken
  // four at a time, heaviest blocks of a group first
  int slot, bh;
  grouped_item(a.B * a.H, nq, 4, bh, slot);
  const int qb = nq - 1 - slot;
  const int h = bh % a.H;
  const int b = bh / a.H;
  const int g = h / (a.H / a.Hkv);
  const int N = a.N;
  const long qbase = ((long)b * a.H + h) * N * D;
  const long kbase = ((long)b * a.Hkv + g) * N * D;
  const uint16_t* qp = (const uint16_t*)a.q + qbase;
  const uint16_t* op = (const uint16_t*)a.o + qbase;
  const uint16_t* dop = (const uint16_t*)a.dout + qbase;
  uint16_t* dqp = (uint16_t*)a.dq + qbase;
  const uint16_t* kp = (const uint16_t*)a.k + kbase;
  const uint16_t* vp = (const uint16_t*)a.v + kbase;

  const int q0 = qb * kBM;
  const int kv_end = CAUSAL ? min(N, q0 + kBM) : N;
  const int n_tiles = (kv_end + kBN - 1) / kBN;
  const int q0w = q0 + 32 * wv;
  const bool wave_live = q0w < N;
  const int qrow = q0w + n32;
  const bool row_ok = qrow < N;

  // Q and dO fragments (B operands: column n32 = row qrow, d = 16c + 8g2 ..
  // +8) and this lane's half of delta = dO . O for the row
  bf16x8 qf[NDC], df[NDC];
  float dsum = 0.f;
#pragma unroll
  for (int c = 0; c < NDC; ++c) {
    u32x4 tq = {0u, 0u, 0u, 0u}, td = tq, to = tq;
    if (row_ok) {
      const long off = (long)qrow * D + 16 * c + 8 * g2;
      tq = ldg16(qp + off);
      td = ldg16(dop + off);
      to = ldg16(op + off);
    }
    qf[c] = as_bf16x8(tq);
    df[c] = as_bf16x8(td);
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      dsum = __builtin_fmaf(bf16_lo(td[x]), bf16_lo(to[x]), dsum);
      dsum = __builtin_fmaf(bf16_hi(td[x]), bf16_hi(to[x]), dsum);
    }
  }
  const float delta = dsum + xor32(dsum);
  const long rowidx = ((long)b * a.H + h) * N + qrow;
  // -LSE in base 2; rows past the end get -inf, so their weights are 0
  const float nl = row_ok ? -a.lse[rowidx] * kLog2e : kNegInf;
  // both row values go to the workspace for the dK/dV kernel
  if (row_ok && g2 == 0) {
    a.delta[rowidx] = delta;
    a.nlse[rowidx] = nl;
  }
  const float c2 = a.c;

  // K/V tile loads: wave instruction i fills LDS bytes (wv + 4i) KB .. +1 KB
  // of a tile; the swizzle is applied through the source address
  uint32_t toff[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int byte = (wv + 4 * i) * 1024 + 16 * lane;
    const int r = byte / ROW;
    const int pc = (byte % ROW) / 16;
    toff[i] = (uint32_t)r * ROW + (uint32_t)(pc ^ swz_kv<D>(r)) * 16u;
  }
  const uint32_t lds0 = lds_addr_of(smem);
  auto load_tile = [&](int j) {
    const int k0 = j * kBN;
    const uint32_t bytes = (uint32_t)(N - k0) * ROW;  // rows k0 .. N-1
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kp + (long)k0 * D, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vp + (long)k0 * D, bytes);
    const uint32_t st = lds0 + (uint32_t)(j & 1) * 2 * TILE + wv * 1024;
#pragma unroll
    for (int i = 0; i < NLD; ++i) lds_dma16(rk, st + 4096 * i, toff[i]);
#pragma unroll
    for (int i = 0; i < NLD; ++i) lds_dma16(rv, st + TILE + 4096 * i, toff[i]);
  };

  // transposing reads of K^T: row offset within the 8-key group and (chunk,
  // byte) of the 4 d values this lane addresses
  const int tr_row = (lane & 15) >> 2;
  const int tr_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int tr_byte = 8 * (lane & 1);

  f32x16 acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;

  // Per-lane LDS byte offsets of the operand reads within a stage.  The
  // swizzle depends only on bits 0..3 of the row, which the lane fixes, so
  // the 32-key block, the 16-row half and K against V are immediate offsets:
  // K (V) fragment (c, kb) at op_off[c] + 32 kb ROW (+ TILE), the two halves
  // of K^T piece (kb, jj, db) at tlo_off[db] / thi_off[db] + (32 kb + 16 jj)
  // ROW.  With the stage a compile-time constant (tiles two at a time, the
  // inner loop unrolled) a tile adds nothing per read; the empty asm keeps
  // each offset in a register of its own.
  uint32_t op_off[NDC], tlo_off[NDB], thi_off[NDB];
  {
    const int r = key_perm(n32);
#pragma unroll
    for (int c = 0; c < NDC; ++c) {
      op_off[c] = (uint32_t)(r * ROW + (((2 * c + g2) ^ swz_kv<D>(r)) << 4));
      asm volatile("" : "+v"(op_off[c]));
    }
    const int kr = 8 * g2 + tr_row;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int ch = 4 * db + tr_chunk;
      tlo_off[db] = (uint32_t)(kr * ROW + ((ch ^ swz_kv<D>(kr)) << 4) + tr_byte);
      thi_off[db] = (uint32_t)((kr + 4) * ROW + ((ch ^ swz_kv<D>(kr + 4)) << 4) + tr_byte);
      asm volatile("" : "+v"(tlo_off[db]), "+v"(thi_off[db]));
    }
  }

  load_tile(0);
  for (int j0 = 0; j0 < n_tiles; j0 += 2)
#pragma unroll
  for (int su = 0; su < 2; ++su) {
    const int j = j0 + su;
    if (j >= n_tiles) break;  // uniform over the workgroup
    wait_vmem();      // this wave's pieces of tile j have landed
    __syncthreads();  // everyone's have; stage (j+1)&1 is free
    if (j + 1 < n_tiles) load_tile(j + 1);
    const int k0 = j * kBN;
    const bool active = wave_live && !(CAUSAL && k0 > q0w + 31);
    if (!active) continue;
    const unsigned char* sk = smem + su * 2 * TILE;
    const unsigned char* sv = sk + TILE;

    __builtin_amdgcn_s_setprio(1);  // products first: other waves fill the gaps with elementwise work
    // S^T = K Q^T and dP^T = V dO^T (keys on the M side, in key_perm order)
    f32x16 s[NKB], dp[NKB];
#pragma unroll
    for (int c = 0; c < NDC; ++c) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const uint32_t off = 32 * kb * ROW + op_off[c];
        const u32x4 kf = *reinterpret_cast<const u32x4*>(sk + off);
        const u32x4 vf = *reinterpret_cast<const u32x4*>(sv + off);
        const f32x16 zero = {};
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf), qf[c], c == 0 ? zero : s[kb], 0, 0, 0);
        dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf), df[c], c == 0 ? zero : dp[kb], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    if ((CAUSAL && k0 + kBN - 1 > q0w) || (k0 + kBN > N)) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = k0 + 32 * kb + acc_key(e, g2);
          if (!(key < N && (!CAUSAL || key <= qrow))) s[kb][e] = kNegInf;
        }
    }
    // dS^T = P^T (dP^T - delta) as bf16 pairs (B operand of the next product)
    uint32_t pk[NKB][8];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      float x[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = exp2_hw(__builtin_fmaf(s[kb][e], c2, nl));
        x[e] = p * (dp[kb][e] - delta);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) pk[kb][e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
    }
    __builtin_amdgcn_s_setprio(1);
    // dQ^T += K^T dS^T; K^T fragments gathered by transposing reads
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const u32x4 pw = {pk[kb][4 * jj], pk[kb][4 * jj + 1], pk[kb][4 * jj + 2], pk[kb][4 * jj + 3]};
        const unsigned char* sb = sk + (32 * kb + 16 * jj) * ROW;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const u32x2 lo = lds_read_tr16(sb + tlo_off[db]);
          const u32x2 hi = lds_read_tr16(sb + thi_off[db]);
          const u32x4 kt = {lo[0], lo[1], hi[0], hi[1]};
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kt), as_bf16x8(pw), acc[db], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
  }

  if (!row_ok) return;
  const float sc = a.scale;
  uint16_t* drow = dqp + (long)qrow * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int jq = 0; jq < 4; ++jq) {
      u32x2 t;
      t[0] = pack_bf16x2(acc[db][4 * jq] * sc, acc[db][4 * jq + 1] * sc);
      t[1] = pack_bf16x2(acc[db][4 * jq + 2] * sc, acc[db][4 * jq + 3] * sc);
      stg8(drow + 32 * db + 8 * jq + 4 * g2, t);
    }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kPairThreads, 2) void bwd_dkdv_kernel(BwdArgs a, int nkb) {
  constexpr int ROW = D * 2;
  constexpr int QT = kBQ * ROW;        // bytes of a Q or dO tile
  constexpr int SLOT = 2 * QT + 2048;  // Q, dO, -LSE log2(e) (1 KB), delta (1 KB)
  constexpr int NSLOT = 3;             // tiles u-1 (second waves), u (first waves), u+1 (loading)
  constexpr int PBUF = kBQ * 32 * 2;   // P of one pair and tile, bf16
  constexpr int NLD = QT / 1024 / 8;   // 1 KB direct loads per wave, tensor and tile
  constexpr int NDC = D / 16;          // k-steps over d of the first products
  constexpr int NDB = D / 32;          // 32-row blocks of d in the accumulators
  static_assert(QT % 8192 == 0, "tile split over eight waves");
  __shared__ __attribute__((aligned(16))) unsigned char smem[NSLOT * SLOT + 2 * 4 * PBUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wv & 3;
  const bool first = wv < 4;  // S, P, dV; the other wave of the pair does dP, dS, dK
  const int n32 = lane & 31;
  const int g2 = lane >> 5;

  // (batch, kv-head, key block); the first key blocks carry the most causal
  // work: all blocks of a kv-head on one XCD, kv-heads taken four at a time,
  // first key blocks of a group first (with the dQ kernel's grouping, the
  // backward measured ~3 % faster than one head at a time)
  int kblk, bg;
  grouped_item(a.B * a.Hkv, nkb, 4, bg, kblk);
  const int g = bg % a.Hkv;
  const int b = bg / a.Hkv;
  const int N = a.N;
  const int grp = a.H / a.Hkv;
  const int k0 = kblk * kKB;
  const int kp0 = k0 + 32 * pair;  // the pair's first key
  const int key = kp0 + n32;       // this lane's key: column of every product
  const bool key_ok = key < N;
  const long kbase = ((long)b * a.Hkv + g) * N * D;

  // B operand of the first product, kept in registers: K^T (first wave) or
  // V^T (second wave); column n32 = key, d = 16c + 8g2 .. +8
  bf16x8 bop[NDC];
  {
    const uint16_t* src = (const uint16_t*)(first ? a.k : a.v) + kbase + (long)key * D + 8 * g2;
#pragma unroll
    for (int c = 0; c < NDC; ++c) {
      u32x4 t = {0u, 0u, 0u, 0u};
      if (key_ok) t = ldg16(src + 16 * c);
      bop[c] = as_bf16x8(t);
    }
  }
  // dV^T (first wave) or dK^T / scale (second wave): row d, column key
  f32x16 acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;

  const int nqb = (N + kBQ - 1) / kBQ;
  const int i0 = CAUSAL ? k0 / kBQ : 0;  // first query tile reaching the block's keys
  const int per_head = nqb - i0;
  const int steps = grp * per_head;      // (query head of the group, query tile)

  // Q/dO tile loads: wave instruction i fills LDS bytes (wv + 8i) KB .. +1 KB;
  // the swizzle is applied through the source address
  uint32_t toff[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int byte = (wv + 8 * i) * 1024 + 16 * lane;
    const int r = byte / ROW;
    const int pc = (byte % ROW) / 16;
    toff[i] = (uint32_t)r * ROW + (uint32_t)(pc ^ swz_kv<D>(r)) * 16u;
  }
  const uint32_t lds0 = lds_addr_of(smem);
  // step u is (query head u / per_head of the group, query tile u % per_head);
  // both are kept as running counters (no division per step): `ld_*` for the
  // tile being loaded, `cur_*` for the tile this wave works on
  // (load_tile is called for u = 0, 1, 2, ... in order)
  int ld_hh = 0, ld_qi = 0, ld_slot = 0;
  auto load_tile = [&]() {
    const int hh = ld_hh;
    const int r0 = (i0 + ld_qi) * kBQ;
    const uint32_t st = lds0 + (uint32_t)ld_slot * SLOT;
    if (++ld_qi == per_head) {
      ld_qi = 0;
      ++ld_hh;
    }
    if (++ld_slot == NSLOT) ld_slot = 0;
    const long rowbase = ((long)b * a.H + g * grp + hh) * N + r0;
    const uint32_t bytes = (uint32_t)(N - r0) * ROW;  // rows r0 .. N-1
    const __amdgpu_buffer_rsrc_t rq = make_rsrc((const uint16_t*)a.q + rowbase * D, bytes);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc((const uint16_t*)a.dout + rowbase * D, bytes);
#pragma unroll
    for (int i = 0; i < NLD; ++i) lds_dma16(rq, st + (wv + 8 * i) * 1024, toff[i]);
#pragma unroll
    for (int i = 0; i < NLD; ++i) lds_dma16(rd, st + QT + (wv + 8 * i) * 1024, toff[i]);
    // -LSE log2(e) and delta of rows r0 .. r0+63, both from the dQ kernel (1 KB
    // of LDS each; lanes past the 64 values land in the unused rest of the
    // region)
    if (wv == 0) lds_dma16(make_rsrc(a.nlse + rowbase, (uint32_t)(N - r0) * 4), st + 2 * QT, 16u * lane);
    if (wv == 1) lds_dma16(make_rsrc(a.delta + rowbase, (uint32_t)(N - r0) * 4), st + 2 * QT + 1024, 16u * lane);
  };

  // transposing reads of dO^T / Q^T: row offset within the 8-query group and
  // (chunk, byte) of the 4 d values this lane addresses
  const int tr_row = (lane & 15) >> 2;
  const int tr_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int tr_byte = 8 * (lane & 1);
  const float c2 = a.c;

  // Step t: the first wave of each pair works on tile t and leaves P in LDS;
  // the second works on tile t-1 with the P its partner left there one step
  // earlier.  One barrier per step orders the DMA of tile t+1 (into the slot
  // tile t-2 used), the P hand-over and the reuse of the two P buffers.
  load_tile();
  int cur_qi = first ? 0 : -1;  // query tile of step u = t (first wave) or t - 1 (second)
  int cur_slot = first ? 0 : NSLOT - 1;  // u % NSLOT
  for (int t = 0; t <= steps; ++t) {
    wait_vmem();      // this wave's pieces of tile t have landed
    __syncthreads();  // everyone's have; tile t-2's slot and P buffer are free
    if (t + 1 < steps) load_tile();
    const int u = first ? t : t - 1;
    const int qi = cur_qi, slot = cur_slot;
    if (++cur_qi == per_head) cur_qi = 0;
    if (++cur_slot == NSLOT) cur_slot = 0;
    if (u < 0 || u >= steps) continue;
    const int r0 = (i0 + qi) * kBQ;
    if (CAUSAL && r0 + kBQ - 1 < kp0) continue;  // every query precedes every key of the pair
    const unsigned char* sq = smem + slot * SLOT;
    const unsigned char* sdo = sq + QT;
    const float* sl = reinterpret_cast<const float*>(sq + 2 * QT);
    const float* sd = sl + 256;
    unsigned char* pbuf = smem + NSLOT * SLOT + ((u & 1) * 4 + pair) * PBUF;

    __builtin_amdgcn_s_setprio(1);  // products first: the partner fills the gaps with elementwise work
    // S = Q K^T (first wave) or dP = dO V^T (second wave), queries on the M
    // side in key_perm order: accumulator element e of block mb is query
    // r0 + 32 mb + acc_key(e, g2), so each lane's 8 values of a 16-query step
    // are 8 consecutive queries (the B operand of the second product)
    const unsigned char* sa = first ? sq : sdo;
    f32x16 s[2];
    // each A fragment is read KW products ahead of its use; the order is
    // pinned (KW reads, then one product and one read at a time) so that the
    // products do not wait on LDS latency
    constexpr int SSTEPS = 2 * NDC;
    constexpr int KW = 2;
    u32x4 af[SSTEPS];
    auto aread = [&](int t) {
      const int c = t / 2, mb = t % 2;
      const int qr = 32 * mb + key_perm(n32);
      return *reinterpret_cast<const u32x4*>(sa + qr * ROW + (((2 * c + g2) ^ swz_kv<D>(qr)) << 4));
    };
#pragma unroll
    for (int t = 0; t < KW; ++t) af[t] = aread(t);
#pragma unroll
    for (int t = 0; t < SSTEPS; ++t) {
      const int c = t / 2, mb = t % 2;
      const f32x16 zero = {};
      s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(af[t]), bop[c], c == 0 ? zero : s[mb], 0, 0, 0);
      if (t + KW < SSTEPS) af[t + KW] = aread(t + KW);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, KW, 0);
#pragma unroll
    for (int t = 0; t < SSTEPS; ++t) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (t + KW < SSTEPS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }

    __builtin_amdgcn_s_setprio(0);
    // B operand of the second product as bf16 pairs: P (first wave) or
    // dS = P (dP - delta) (second wave); P goes through LDS lane for lane
    uint32_t w[2][8];
    if (first) {
      const bool masked = (CAUSAL && r0 < kp0 + 31) || (r0 + kBQ > N);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        f32x4 lv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          lv[j] = *reinterpret_cast<const f32x4*>(sl + 32 * mb + 16 * (j >> 1) + 8 * g2 + 4 * (j & 1));
        float p[16];
        // the mask test stays outside the element loop: one uniform branch per
        // block, selects inside it
        if (masked) {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int row = r0 + 32 * mb + acc_key(e, g2);
            const float x = (row < N && (!CAUSAL || key <= row)) ? s[mb][e] : kNegInf;
            p[e] = exp2_hw(__builtin_fmaf(x, c2, lv[e >> 2][e & 3]));
          }
        } else {
#pragma unroll
          for (int e = 0; e < 16; ++e) p[e] = exp2_hw(__builtin_fmaf(s[mb][e], c2, lv[e >> 2][e & 3]));
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) w[mb][i] = pack_bf16x2(p[2 * i], p[2 * i + 1]);
        *reinterpret_cast<u32x4*>(pbuf + mb * 2048 + 16 * lane) = u32x4{w[mb][0], w[mb][1], w[mb][2], w[mb][3]};
        *reinterpret_cast<u32x4*>(pbuf + mb * 2048 + 1024 + 16 * lane) = u32x4{w[mb][4], w[mb][5], w[mb][6], w[mb][7]};
      }
    } else {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        f32x4 dv4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          dv4[j] = *reinterpret_cast<const f32x4*>(sd + 32 * mb + 16 * (j >> 1) + 8 * g2 + 4 * (j & 1));
        const u32x4 p0 = *reinterpret_cast<const u32x4*>(pbuf + mb * 2048 + 16 * lane);
        const u32x4 p1 = *reinterpret_cast<const u32x4*>(pbuf + mb * 2048 + 1024 + 16 * lane);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t pw = i < 4 ? p0[i] : p1[i - 4];
          const int e0 = 2 * i, e1 = 2 * i + 1;
          const float x0 = bf16_lo(pw) * (s[mb][e0] - dv4[e0 >> 2][e0 & 3]);
          const float x1 = bf16_hi(pw) * (s[mb][e1] - dv4[e1 >> 2][e1 & 3]);
          w[mb][i] = pack_bf16x2(x0, x1);
        }
      }
    }

    __builtin_amdgcn_s_setprio(1);
    // dV^T += dO^T P (first wave) or dK^T += Q^T dS (second wave); dO^T and
    // Q^T gathered by transposing reads
    const unsigned char* sb = first ? sdo : sq;
    // fragments read PW products ahead, pinned as above
    constexpr int PSTEPS = 4 * NDB;
    constexpr int PW = 2;
    u32x4 bt[PSTEPS];
    auto bread = [&](int t) {
      const int mb = t / (2 * NDB), jj = (t / NDB) % 2, db = t % NDB;
      const int qrow = 32 * mb + 16 * jj + 8 * g2 + tr_row;
      const int ch = 4 * db + tr_chunk;
      const u32x2 lo = lds_read_tr16(sb + qrow * ROW + ((ch ^ swz_kv<D>(qrow)) << 4) + tr_byte);
      const u32x2 hi = lds_read_tr16(sb + (qrow + 4) * ROW + ((ch ^ swz_kv<D>(qrow + 4)) << 4) + tr_byte);
      return u32x4{lo[0], lo[1], hi[0], hi[1]};
    };
#pragma unroll
    for (int t = 0; t < PW; ++t) bt[t] = bread(t);
#pragma unroll
    for (int t = 0; t < PSTEPS; ++t) {
      const int mb = t / (2 * NDB), jj = (t / NDB) % 2, db = t % NDB;
      const u32x4 pw = {w[mb][4 * jj], w[mb][4 * jj + 1], w[mb][4 * jj + 2], w[mb][4 * jj + 3]};
      acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(bt[t]), as_bf16x8(pw), acc[db], 0, 0, 0);
      if (t + PW < PSTEPS) bt[t + PW] = bread(t + PW);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * PW, 1);
#pragma unroll
    for (int t = 0; t < PSTEPS; ++t) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      if (t + PW < PSTEPS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
    }
    __builtin_amdgcn_s_setprio(0);
  }

  if (!key_ok) return;
  // accumulator row 8 jq + 4 g2 + r of block db is d = 32 db + 8 jq + 4 g2 + r of this key
  const float f = first ? 1.f : a.scale;
  uint16_t* dst = (uint16_t*)(first ? a.dv : a.dk) + kbase + (long)key * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int jq = 0; jq < 4; ++jq) {
      u32x2 t;
      t[0] = pack_bf16x2(acc[db][4 * jq] * f, acc[db][4 * jq + 1] * f);
      t[1] = pack_bf16x2(acc[db][4 * jq + 2] * f, acc[db][4 * jq + 3] * f);
      stg8(dst + 32 * db + 8 * jq + 4 * g2, t);
    }
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_one(const BwdArgs& a, hipStream_t stream) {
  const int nq = (a.N + kBM - 1) / kBM;
  const long g1 = (long)nq * a.H * a.B;
  const int nkb = (a.N + kKB - 1) / kKB;
  const long g2 = (long)nkb * a.Hkv * a.B;
  if (g1 <= 0) return hipSuccess;
  if (g1 > 0x7fffffffL || g2 > 0x7fffffffL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)g1), dim3(kThreads), 0, stream, a, nq);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)g2), dim3(kPairThreads), 0, stream, a, nkb);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream) {
  if (a.d == 128) return a.causal ? launch_bwd_one<128, true>(a, stream) : launch_bwd_one<128, false>(a, stream);
  if (a.d == 64) return a.causal ? launch_bwd_one<64, true>(a, stream) : launch_bwd_one<64, false>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace fattn
