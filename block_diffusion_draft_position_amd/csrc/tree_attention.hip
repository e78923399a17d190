// Grouped-query tree attention: every node of the draft tree attends to the prefix
// KV cache plus its own ancestors, all nodes in one pass (DDTree page "策展 · X
// (Twitter)": section 核心創新 for the ancestor-only mask, 運作流程 step 3 for
// scoring the whole tree in one target forward).
//
// bf16 path (the hot path)
//   For one sequence s and KV head g the R = G * N query rows (rows ordered node-major:
//   r = n * G + h % G) share every key.  A workgroup owns a block of rows (32 per
//   wave) and one split of the keys; it streams that split's K/V through LDS once, in
//   tiles of 64 keys, and all its waves reuse each tile.  Splits are the prefix cut
//   into chunks, plus one more split holding the N tree keys, which are masked by the
//   ancestor bitmask.  Each split leaves an unnormalised partial (O, running max, sum)
//   per row; attn_combine merges them in log-sum-exp form (deterministic, no atomics).
//
//   attn_partial_bf16 (D = 32, 64): per wave and 32-key half-tile, with the MFMA
//   v_mfma_f32_32x32x16_bf16 and register-staged tiles:
//     S^T[key][query] = K[key][:] . Q[query][:]          (D/16 MFMAs)
//     O^T[d][query]  += V^T[d][key] . P^T[key][query]     (2 * D/32 MFMAs)
//   Computing the transposes puts one query column in each lane (lanes l and l+32
//   share a query), so the softmax max/sum is in-lane plus one cross-half exchange,
//   and the S^T accumulator registers are already the B operand of the PV product
//   (the PV contraction visits the half-tile's keys in the permuted order
//   k(b, 8h + j) = 16b + 8(j / 4) + 4h + j % 4, and V^T is read in that order).
//   V is stored transposed in LDS (d-major) so that operand is two 8-byte reads.
//   Online softmax runs in base 2 with scale * log2(e) folded into one multiply.
//
//   attn_d128 (D = 128): 32 query rows per wave as two blocks of 16, K/V tiles moved
//   global -> LDS by DMA through a 2-stage ring, v_mfma_f32_16x16x32_bf16 for both
//   products, V^T read with the transposing LDS load (details at the kernel).
//
//   Partials are written with nontemporal stores: the combine reads each once, and
//   keeping them out of the L2 keeps the end-of-kernel cache writeback short.
//
// fp32 path: one wave per query row over all of its keys (no splits), VALU only.
#include <hip/hip_ext.h>
#include <math.h>

#include "ddt_internal.h"

namespace ddt {
namespace {

typedef __bf16 bf16_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

constexpr int kTile = 64;         // keys per LDS tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int D>
struct Lds {
  static constexpr int kPitch = D + 8;        // K tile row pitch (bf16 elements)
  static constexpr int vPitch = kTile + 4;    // V^T tile row pitch (bf16 elements)
  static constexpr int kElems = kTile * kPitch;
  static constexpr int vElems = D * vPitch;
  static constexpr size_t bytes = sizeof(bf16_t) * (kElems + vElems);
};

__device__ __forceinline__ uint32_t pack2(bf16_t a, bf16_t b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

struct Unit {
  int s, g, c, rg;
};

// Workgroup -> (unit, row group).  Row groups of one unit are 8 workgroups apart,
// so they land on the same XCD (workgroups are dealt to the 8 XCDs round robin)
// and share that XCD's L2 for the unit's K/V.  The split index varies slowest, so
// consecutive units are different (sequence, KV head) pairs of equal kind and the
// prefix splits spread over all XCDs (tree splits, which are short, come last).
__device__ __forceinline__ bool decode_block(int Hkv, int nsplit_tot, int row_groups, int units,
                                             Unit& u) {
  const int blk = blockIdx.x;
  const int x8 = blk & 7;
  const int rest = blk >> 3;
  u.rg = rest % row_groups;
  const int un = (rest / row_groups) * 8 + x8;
  if (un >= units) return false;
  const int nsg = units / nsplit_tot;  // sequences x KV heads
  u.c = un / nsg;
  const int sg = un % nsg;
  u.g = sg % Hkv;
  u.s = sg / Hkv;
  return true;
}

// As decode_block, for attn_d128 with a last row group of at most 32 rows among at least
// eight (rem_last): those groups run as two short streams and take no part in the L2
// sharing of a unit's full groups, so all of them come after every other workgroup.  The
// full groups keep the dispatch pattern above, and the remainders fill the CUs that the
// grid's tail leaves idle.  (With fewer groups the remainders are too large a share of
// the grid to hide in its tail: C4, five groups, ran 15% slower that way; C2 no faster.)
__device__ __forceinline__ bool decode_block_rl(int Hkv, int nsplit_tot, int row_groups, int units,
                                                bool rem_last, Unit& u) {
  if (!rem_last) return decode_block(Hkv, nsplit_tot, row_groups, units, u);
  const int blk = blockIdx.x;
  const int full = row_groups - 1;
  const int nfull = (units + 7) / 8 * 8 * full;
  int un;
  if (blk < nfull) {
    const int rest = blk >> 3;
    u.rg = rest % full;
    un = (rest / full) * 8 + (blk & 7);
  } else {
    u.rg = full;
    un = blk - nfull;
  }
  if (un >= units) return false;
  const int nsg = units / nsplit_tot;
  u.c = un / nsg;
  const int sg = un % nsg;
  u.g = sg % Hkv;
  u.s = sg / Hkv;
  return true;
}

template <int D, int NW>
__global__ void __launch_bounds__(NW * 64)
attn_partial_bf16(const bf16_t* __restrict__ q, const bf16_t* __restrict__ kc,
                  const bf16_t* __restrict__ vc, Prefix pre,
                  const bf16_t* __restrict__ kt, const bf16_t* __restrict__ vt,
                  const uint32_t* __restrict__ mask, const int32_t* __restrict__ num_nodes,
                  int N, int Hq, int Hkv, int G, int R, int W, int rows_pad, int nsplit,
                  int64_t chunk, int units, int row_groups, float scale_log2,
                  float* __restrict__ opart, float2* __restrict__ mlpart) {
  constexpr int NT = NW * 64;
  constexpr int KSTEPS = D / 16;   // MFMA k-steps over the head dim
  constexpr int DBLK = D / 32;     // 32-row blocks of O^T
  constexpr int DCH = D / 8;       // 16-byte chunks per key row
  constexpr int KCH = kTile * DCH;          // K chunks per tile
  constexpr int VCH = (kTile / 2) * DCH;    // V key-pair chunks per tile
  constexpr int KPT = (KCH + NT - 1) / NT;  // per thread
  constexpr int VPT = (VCH + NT - 1) / NT;
  using L = Lds<D>;

  extern __shared__ __align__(16) unsigned char smem_raw[];
  bf16_t* Ks = reinterpret_cast<bf16_t*>(smem_raw);
  bf16_t* Vs = Ks + L::kElems;

  Unit u;
  if (!decode_block(Hkv, nsplit + 1, row_groups, units, u)) return;
  const int tid = threadIdx.x;
  const int wave = tid / 64;
  const int lane = tid % 64;
  const int h2 = lane / 32;     // lane half
  const int l32 = lane % 32;

  const int nn = num_nodes[u.s];
  const int64_t p0 = pre.start(u.s);
  const int64_t P = kc ? pre.length(u.s) : 0;
  const int64_t kstride = (int64_t)Hkv * D;   // elements between consecutive keys
  const bool tree = u.c == nsplit;
  int64_t lo, hi;
  const bf16_t* kb;
  const bf16_t* vb;
  if (!tree) {
    const int64_t nvalid = P > 0 ? min<int64_t>(nsplit, (P + chunk - 1) / chunk) : 0;
    if (u.c >= nvalid) return;
    lo = (int64_t)u.c * chunk;
    hi = (u.c == nvalid - 1) ? P : lo + chunk;
    kb = kc + (p0 * Hkv + u.g) * D;
    vb = vc + (p0 * Hkv + u.g) * D;
  } else {
    lo = 0;
    hi = nn;
    kb = kt + ((int64_t)u.s * N * Hkv + u.g) * D;
    vb = vt + ((int64_t)u.s * N * Hkv + u.g) * D;
  }

  // this lane's query row
  const int row = (u.rg * NW + wave) * 32 + l32;
  const int node = row / G;
  const bool row_ok = row < R && node < nn;
  const int head = u.g * G + (row % G);

  // Q fragments: B operand of S^T, lane holds Q[row][16kk + 8h2 .. +8]
  bf16x8 qf[KSTEPS];
  {
    const bf16_t* qrow = q + (((int64_t)u.s * N + node) * Hq + head) * D;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      if (row_ok)
        qf[kk] = *reinterpret_cast<const bf16x8*>(qrow + kk * 16 + h2 * 8);
      else
        qf[kk] = bf16x8{};
    }
  }
  const uint32_t* mrow = mask + ((int64_t)u.s * N + (row_ok ? node : 0)) * W;

  f32x16 oacc[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY;  // running max, base-2 units, same in both lane halves
  float l_run = 0.f;        // this lane's share of the running sum

  // register staging of the next tile
  uint4 kreg[KPT];
  uint4 vreg[VPT][2];
  auto load_tile = [&](int64_t t0) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int qi = tid + i * NT;
      const int key = qi / DCH, dc = qi % DCH;
      kreg[i] = make_uint4(0, 0, 0, 0);
      if (qi < KCH && t0 + key < hi)
        kreg[i] = *reinterpret_cast<const uint4*>(kb + (t0 + key) * kstride + dc * 8);
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int qi = tid + i * NT;
      const int kp = qi % (kTile / 2), dc = qi / (kTile / 2);
      vreg[i][0] = make_uint4(0, 0, 0, 0);
      vreg[i][1] = make_uint4(0, 0, 0, 0);
      if (qi < VCH) {
        if (t0 + 2 * kp < hi)
          vreg[i][0] = *reinterpret_cast<const uint4*>(vb + (t0 + 2 * kp) * kstride + dc * 8);
        if (t0 + 2 * kp + 1 < hi)
          vreg[i][1] = *reinterpret_cast<const uint4*>(vb + (t0 + 2 * kp + 1) * kstride + dc * 8);
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int qi = tid + i * NT;
      if (qi < KCH) {
        const int key = qi / DCH, dc = qi % DCH;
        *reinterpret_cast<uint4*>(Ks + key * L::kPitch + dc * 8) = kreg[i];
      }
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int qi = tid + i * NT;
      if (qi < VCH) {
        const int kp = qi % (kTile / 2), dc = qi / (kTile / 2);
        const uint32_t a[4] = {vreg[i][0].x, vreg[i][0].y, vreg[i][0].z, vreg[i][0].w};
        const uint32_t b[4] = {vreg[i][1].x, vreg[i][1].y, vreg[i][1].z, vreg[i][1].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // d = dc*8 + 2e (low halves) and 2e+1 (high halves): pair keys 2kp, 2kp+1
          const uint32_t lo16 = (a[e] & 0xffffu) | (b[e] << 16);
          const uint32_t hi16 = (a[e] >> 16) | (b[e] & 0xffff0000u);
          *reinterpret_cast<uint32_t*>(Vs + (dc * 8 + 2 * e) * L::vPitch + 2 * kp) = lo16;
          *reinterpret_cast<uint32_t*>(Vs + (dc * 8 + 2 * e + 1) * L::vPitch + 2 * kp) = hi16;
        }
      }
    }
  };

  const int64_t ntiles = (hi - lo + kTile - 1) / kTile;
  if (ntiles > 0) load_tile(lo);
  for (int64_t t = 0; t < ntiles; ++t) {
    const int64_t t0 = lo + t * kTile;
    __syncthreads();  // previous tile's readers are done
    store_tile();
    __syncthreads();
    if (t + 1 < ntiles) load_tile(t0 + kTile);  // in flight during the math below

    // ---- S^T = K . Q^T for two 32-key halves
    f32x16 sacc[2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      sacc[kh] = f32x16{};
      const bf16_t* krow = Ks + (kh * 32 + l32) * L::kPitch + h2 * 8;
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + kk * 16);
        sacc[kh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], sacc[kh], 0, 0, 0);
      }
    }
    // ---- scale, mask, tile max
    uint32_t mw0 = 0xffffffffu, mw1 = 0xffffffffu;
    if (tree) {
      const int w0 = (int)(t0 >> 5);
      mw0 = (w0 < W) ? mrow[w0] : 0u;
      mw1 = (w0 + 1 < W) ? mrow[w0 + 1] : 0u;
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kin = kh * 32 + 8 * (i / 4) + 4 * h2 + (i % 4);   // key within tile
        bool ok = t0 + kin < hi;
        if (tree) ok = ok && (((kh ? mw1 : mw0) >> (kin & 31)) & 1u);
        const float v = ok ? sacc[kh][i] * scale_log2 : -INFINITY;
        sacc[kh][i] = v;
        tmax = fmaxf(tmax, v);
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < DBLK; ++i) oacc[i] *= alpha;

    // ---- P = exp2(S - m) as bf16 B operands; row sums
    bf16x8 pb[2][2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float p = __builtin_amdgcn_exp2f(sacc[kh][8 * b + j] - m_use);
          l_run += p;
          pb[kh][b][j] = (bf16_t)p;
        }
      }
    }
    // ---- O^T += V^T . P^T
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
      const bf16_t* vrow = Vs + (db * 32 + l32) * L::vPitch + 4 * h2;
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const bf16x4 v0 = *reinterpret_cast<const bf16x4*>(vrow + kh * 32 + 16 * b);
          const bf16x4 v1 = *reinterpret_cast<const bf16x4*>(vrow + kh * 32 + 16 * b + 8);
          const bf16x8 a = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kh][b], oacc[db], 0, 0, 0);
        }
      }
    }
  }

  // ---- partial results of this split
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (row < R) {
    const int64_t urow = (((int64_t)u.s * Hkv + u.g) * (nsplit + 1) + u.c) * rows_pad + row;
    float* orow = opart + urow * D;
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int d = db * 32 + 8 * qq + 4 * h2;
        __builtin_nontemporal_store(
            f32x4{oacc[db][4 * qq], oacc[db][4 * qq + 1], oacc[db][4 * qq + 2], oacc[db][4 * qq + 3]},
            reinterpret_cast<f32x4*>(orow + d));
      }
    }
    if (h2 == 0) __builtin_nontemporal_store(f32x2{m_run, l_tot}, reinterpret_cast<f32x2*>(mlpart + urow));
  }
}

// ---------------------------------------------------------------- bf16, D = 128 (gfx950 path)
// Same decomposition as attn_partial_bf16, rebuilt around gfx950 features:
//   * K and V tiles (64 keys) go global -> LDS with buffer_load_dwordx4 ... lds, no
//     registers in between, into a 2-stage ring: tile t + 1 is issued right after
//     the barrier that opens tile t, so one tile is in flight while one is consumed.
//     One barrier per tile suffices: the stage refilled after barrier t was last
//     read in tile t - 1, which every wave finished before arriving at barrier t.
//     A 256-byte key row keeps its sixteen
//     16-byte chunks XOR-swizzled (chunk c of key k at slot c ^ swz(k)) so that
//     both the K reads and the transposed V reads are free of bank conflicts.
//   * V stays row-major; the PV operand V^T is read with ds_read_b64_tr_b16, which
//     hands each lane of a 16-lane group one head-dim column of a 4-key block.
//   * v_mfma_f32_16x16x32_bf16 with 32 query rows per wave (two 16-row blocks that
//     share every K/V fragment read from LDS).  QK^T runs head-dim step outermost, so
//     eight independent accumulators alternate, and the next step's K fragments are read
//     while a step's MFMAs run; PV goes through head-dim blocks in pairs, the next
//     pair's V fragments read while a pair's MFMAs run (a wave waits on LDS three or
//     four times per product instead of eight).
//   * The per-sequence bounds, the split's length and the tile index live in scalar
//     registers, a full tile's loads need one lane offset in all, and the rare paths (a
//     split's partial last tile, the lazy rescale) are real branches: left to itself
//     the compiler turned them into selects executed on every tile.  The kernel fits
//     in 256 registers without spilling at every workgroup width.
//   * The running max is raised only when a tile's max exceeds it by more than
//     2^8; otherwise O and l are not rescaled (p <= 2^8 stays exact in fp32/bf16).
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kStages = 2;
constexpr int kTileBytes = kTile * 128 * 2;      // one K or V tile, D = 128
constexpr float kTau = 8.f;                      // lazy-rescale slack (base-2 units)

// The ring: two stages of one K and one V tile each, 64 KB, so two workgroups fit in a
// CU's LDS.  Two co-resident workgroups run their phases (LDS reads, MFMA, the exp of
// the softmax) out of step with each other, which overlaps them on every SIMD better
// than deeper prefetch within one workgroup does (measured on C2, C3 and C4 shapes).
// One statically allocated K and V buffer per stage.  Separate objects let
// the compiler see that a stage being read does not alias the stages still being
// filled, so it keeps the explicit per-stage vmcnt waits instead of draining all
// outstanding loads before every LDS read.
__shared__ __align__(16) unsigned char g_ring_k0[kTileBytes], g_ring_v0[kTileBytes];
__shared__ __align__(16) unsigned char g_ring_k1[kTileBytes], g_ring_v1[kTileBytes];

template <int ST>
__device__ __forceinline__ unsigned char* ring_k() {
  if constexpr (ST == 0) return g_ring_k0;
  if constexpr (ST == 1) return g_ring_k1;
}
template <int ST>
__device__ __forceinline__ unsigned char* ring_v() {
  if constexpr (ST == 0) return g_ring_v0;
  if constexpr (ST == 1) return g_ring_v1;
}

// Slot swizzle of a key row (a bijection on 0..15): the sixteen K rows read by one
// 16-lane group land in sixteen different 16-byte slots, and the four rows of a
// transposed V read get slot offsets that differ in bits 1-3 with bit 0 equal, so
// with the two chunks (c, c ^ 1) they fill sixteen different slots per 32 lanes.
// (Measured: a variant aimed at 32 banks doubled the bank-conflict cycles.)
__device__ __forceinline__ int64_t rfl64(int64_t v) {
  const int lo32 = __builtin_amdgcn_readfirstlane((int)(v & 0xffffffff));
  const int hi32 = __builtin_amdgcn_readfirstlane((int)(v >> 32));
  return (int64_t)(((uint64_t)(uint32_t)hi32 << 32) | (uint32_t)lo32);
}

constexpr int kRsrcWord3 = 0x00020000;  // gfx9-family raw buffer: 32-bit data format

__device__ __forceinline__ int swz(int key) { return ((key & 7) << 1) | ((key >> 3) & 1); }

template <int NW>
__global__ void __launch_bounds__(NW * 64, NW <= 4 ? 2 : 1)
attn_d128(const bf16_t* __restrict__ q, const bf16_t* __restrict__ kc,
          const bf16_t* __restrict__ vc, Prefix pre,
          const bf16_t* __restrict__ kt, const bf16_t* __restrict__ vt,
          const uint32_t* __restrict__ mask, const int32_t* __restrict__ num_nodes,
          int N, int Hq, int Hkv, int G, int R, int W, int rows_pad, int nsplit,
          int64_t chunk, int units, int row_groups, float scale_log2,
          float* __restrict__ opart, float2* __restrict__ mlpart) {
  constexpr int D = 128;

  // the last row group of each unit holds at most 32 rows (see solo below), one of many
  const bool rem_last = NW >= 2 && row_groups >= 8 && R - (row_groups - 1) * NW * 32 <= 32;
  Unit u;
  if (!decode_block_rl(Hkv, nsplit + 1, row_groups, units, rem_last, u)) return;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);  // uniform: kept in an SGPR
  __builtin_assume(wave < NW);
  const int lane = tid % 64;
  const int g4 = lane / 16;   // 16-lane group
  const int l16 = lane % 16;

  // per-sequence bounds, uniform across the workgroup: kept in scalar registers so that
  // the tile loop's bounds, tail tests and branches are scalar
  const int nn = __builtin_amdgcn_readfirstlane(num_nodes[u.s]);
  const int64_t p0 = rfl64(pre.start(u.s));
  const int64_t P = kc ? rfl64(pre.length(u.s)) : 0;
  const int64_t kstride = (int64_t)Hkv * D;
  const bool tree = u.c == nsplit;
  // A remainder group (the last row group of a unit) whose rows fit in one wave: the
  // barrier-paced ring would keep one tile in flight for a single wave's work.  There
  // waves 0 and 1 instead stream alternate tiles alone, each through one ring stage
  // with no barrier, both for the same rows, and merge their two partials at the end;
  // a wave whose rows fit in 16 computes one query block.  Prefix splits only.
  const int grp_rows = R - u.rg * NW * 32;
  const bool solo = NW >= 2 && !tree && grp_rows <= 32;
  const bool one_qb = grp_rows <= 16;
  const int wslot = solo ? 0 : wave;
  // otherwise a wave whose 32 rows all lie past R (the last row group of a unit holds
  // only the remainder) issues its share of the tile loads and meets the barriers, no more
  const bool live = solo ? wave < 2 : (u.rg * NW + wave) * 32 < R;
  int64_t lo, hi;
  const bf16_t* kb;
  const bf16_t* vb;
  if (!tree) {
    const int64_t nvalid = P > 0 ? min<int64_t>(nsplit, (P + chunk - 1) / chunk) : 0;
    if (u.c >= nvalid) return;
    lo = (int64_t)u.c * chunk;
    hi = (u.c == nvalid - 1) ? P : lo + chunk;
    kb = kc + ((p0 + lo) * Hkv + u.g) * D;
    vb = vc + ((p0 + lo) * Hkv + u.g) * D;
  } else {
    lo = 0;
    hi = nn;
    kb = kt + ((int64_t)u.s * N * Hkv + u.g) * D;
    vb = vt + ((int64_t)u.s * N * Hkv + u.g) * D;
  }
  // the split's key count and tiles, uniform (readfirstlane: else the compiler keeps
  // them in vector registers and every per-tile test becomes a divergent branch)
  const int64_t span = rfl64(hi - lo);
  const int ntiles = __builtin_amdgcn_readfirstlane((int)((span + kTile - 1) / kTile));

  // ---- the loads of tile t into ring stage ST: 32 instructions of 1 KB (4 key rows),
  // 16 for K then 16 for V, dealt round robin to the waves.  Rows past the split
  // (last tile) re-read the split's last row and are masked later.
  // Tile loads go through buffer resources based at the tile's first row (one for K, one
  // for V; rebuilt per tile with scalar arithmetic): a scalar byte offset carries the
  // load's row block, a 32-bit lane offset the rest, so no 64-bit address is formed per
  // lane and offsets stay below 64 rows whatever the split's length.  A load's key row
  // is 4 * (i & 15) + g4 and its swizzle splits into disjoint bits, 2 g4 from the lane
  // and 8 (i & 1) + (i >> 1 & 1) from the (uniform) load index; a row is 256-byte
  // aligned, so the lane offset of a full tile's load is one lane base XOR a uniform
  // constant.  (The bases pass through readfirstlane: the compiler then knows them to
  // be uniform, else it wraps every load in a loop over the wave's distinct resources.)
  const unsigned char* kbu = (const unsigned char*)rfl64((int64_t)kb);
  const unsigned char* vbu = (const unsigned char*)rfl64((int64_t)vb);
  const uint32_t rowb = (uint32_t)kstride * 2;  // bytes per key row, a multiple of 256
  const uint32_t lane_base = (uint32_t)g4 * rowb + (uint32_t)((l16 ^ (2 * g4)) * 16);
  // NI waves share a tile's loads (NI = NW), or wave 0 or 1 alone (NI = 1) issues all 32
  auto issue = [&]<int ST, int NI = NW>(int t_) {
    constexpr int NL = (32 + NI - 1) / NI;
    const int wi = NI == 1 ? 0 : wave;
    const int t = __builtin_amdgcn_readfirstlane(t_);
    const int64_t t0 = (int64_t)t * kTile;  // from lo
    const int64_t tb = t0 * rowb;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(kbu + tb), (short)0, -1, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(vbu + tb), (short)0, -1, kRsrcWord3);
    if (t0 + kTile <= span) {
      if constexpr (16 % NI == 0) {
        // NI divides 16: load j is wave wi's row block rb = wi + NI (j mod 16 / NI), of K
        // for j < 16 / NI and of V after, so the operand is known at compile time and
        // the row offset, destination and swizzle are the wave's own plus constants
        // (recomputed from the wave index per tile they took ~100 scalar instructions
        // and spilled scalar registers)
        constexpr int PER = 16 / NI;
#pragma unroll
        for (int j = 0; j < NL; ++j) {
          const bool isv = j >= PER;
          const int rb = wi + NI * (j % PER);
          unsigned char* dst = (isv ? ring_v<ST>() : ring_k<ST>()) + rb * 1024;
          const uint32_t x = 16u * (8u * (rb & 1) + ((rb >> 1) & 1));
          uint32_t so = (uint32_t)(4 * rb) * rowb;
          if constexpr (NI == 1) so = __builtin_amdgcn_readfirstlane(so);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(isv ? rv : rk, (lds_void*)dst, 16, lane_base ^ x,
                                                   so, 0, 0);
        }
      } else {
#pragma unroll
        for (int j = 0; j < NL; ++j) {
          const int i = (wi + j * NI) & 31;
          const bool isv = i >= 16;
          unsigned char* dst = (isv ? ring_v<ST>() : ring_k<ST>()) + (i & 15) * 1024;
          const uint32_t x = 16u * (8u * (i & 1) + ((i >> 1) & 1));
          __builtin_amdgcn_raw_ptr_buffer_load_lds(isv ? rv : rk, (lds_void*)dst, 16, lane_base ^ x,
                                                   (uint32_t)(4 * (i & 15)) * rowb, 0, 0);
        }
      }
    } else {
      // the split's last, partial tile: rows past the split re-read its last row.  (The
      // lane terms pass through an empty asm so that the per-load offsets are formed
      // here, not hoisted out of the tile loop and kept live.)
      asm volatile("" ::: "memory");
      int gl = g4;
      uint32_t lchunk = (uint32_t)((l16 ^ (2 * g4)) * 16);
      asm volatile("" : "+v"(gl), "+v"(lchunk));
      const int last = (int)(span - 1 - t0);
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        const int i = (wi + j * NI) & 31;
        const bool isv = i >= 16;
        const int key = min(4 * (i & 15) + gl, last);
        const uint32_t off = (uint32_t)key * rowb + (lchunk ^ (16u * (8u * (i & 1) + ((i >> 1) & 1))));
        unsigned char* dst = (isv ? ring_v<ST>() : ring_k<ST>()) + (i & 15) * 1024;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(isv ? rv : rk, (lds_void*)dst, 16, off, 0, 0, 0);
      }
    }
  };

  // ---- this lane's two query rows (blocks of 16) and their Q fragments (B operand)
  int rowq[2], nodeq[2];
  bool okq[2];
  bf16x8 qf[2][4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    rowq[qb] = (u.rg * NW + wslot) * 32 + qb * 16 + l16;
    nodeq[qb] = rowq[qb] / G;
    okq[qb] = rowq[qb] < R && nodeq[qb] < nn;
    const int head = u.g * G + (rowq[qb] % G);
    const bf16_t* qrow = q + (((int64_t)u.s * N + nodeq[qb]) * Hq + head) * D;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      qf[qb][kk] = okq[qb] ? *reinterpret_cast<const bf16x8*>(qrow + kk * 32 + g4 * 8) : bf16x8{};
  }
  // the sequence's mask (uniform base) and this lane's two rows in it, as 32-bit byte
  // offsets: the word loads take the scalar-base form
  const unsigned char* mseq = (const unsigned char*)(mask + (int64_t)u.s * N * W);
  const uint32_t mrow0 = (uint32_t)((okq[0] ? nodeq[0] : 0) * W) * 4u;
  const uint32_t mrow1 = (uint32_t)((okq[1] ? nodeq[1] : 0) * W) * 4u;

  // per-lane LDS read offsets (see the reads below)
  int kofs[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) kofs[kk] = l16 * 256 + (((4 * kk + g4) ^ swz(l16)) << 4);
  const int vrow = 4 * g4 + l16 / 4;   // key row within a 32-key half (and +16)
  const int vsw = swz(vrow);
  const int vsw_hi = vsw & 14;
  const int vsw_lo = ((l16 & 3) >> 1) ^ (vsw & 1);
  const int vbase = vrow * 256 + (l16 & 1) * 8;

  f32x4 oacc[2][8];
  f32x4 lacc[2];  // row sums of P, from an MFMA against an all-ones block
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
    for (int db = 0; db < 8; ++db) oacc[qb][db] = f32x4{};
    lacc[qb] = f32x4{};
  }
  float m_run[2] = {-INFINITY, -INFINITY};
  bf16x8 ones;
#pragma unroll
  for (int j = 0; j < 8; ++j) ones[j] = (bf16_t)1.f;

  // ---- the math of tile t from ring stage ST, for QB query blocks of 16 rows
  auto math = [&]<int ST, int QB>(int t, const uint32_t (&w)[2][2]) {
    // Per-lane offsets are re-materialised in every step (an empty asm hides their
    // loop invariance); otherwise the compiler keeps one copy per ring stage live.
    int kof[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      kof[kk] = kofs[kk];
      asm volatile("" : "+v"(kof[kk]));
    }
    int vb_ = vbase, vhi = vsw_hi, vlo = vsw_lo;
    asm volatile("" : "+v"(vb_), "+v"(vhi), "+v"(vlo));
    const unsigned char* Ks = ring_k<ST>();
    const unsigned char* Vs = ring_v<ST>();
    const int64_t t0 = lo + (int64_t)t * kTile;
    const int rem = __builtin_amdgcn_readfirstlane((int)span - t * kTile);  // keys left; masks if < 64

    // ---- S^T = K . Q^T  (4 key blocks x 2 query blocks), head-dim step kk outermost:
    // eight independent accumulators per step, and step kk + 1's four K fragments are
    // read while step kk's eight MFMAs run.  Key kb4*16 + l16 has the swizzle of l16, so
    // the lane's read offsets are kofs[kk] + kb4 * 4096.
    f32x4 sacc[2][4];
    bf16x8 kf[2][4];
    auto kread = [&](int kk, bf16x8 (&f)[4]) {
#pragma unroll
      for (int kb4 = 0; kb4 < 4; ++kb4) f[kb4] = *reinterpret_cast<const bf16x8*>(Ks + kof[kk] + kb4 * 4096);
    };
    kread(0, kf[0]);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kk + 1 < 4) kread(kk + 1, kf[(kk + 1) & 1]);
#pragma unroll
      for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          sacc[qb][kb4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kk & 1][kb4], qf[qb][kk],
                                                                  kk == 0 ? f32x4{} : sacc[qb][kb4], 0, 0, 0);
    }
    // order: the first two steps' reads, then per step QB MFMAs per read of the next
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int kk = 0; kk < 3; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);
      }
    __builtin_amdgcn_sched_group_barrier(0x008, 4 * QB, 0);
    __builtin_amdgcn_sched_barrier(0);  // keep the phases apart: bounded register use
    // ---- masks: ragged tail, and in the tree split the ancestor bits
    if (tree) {
      // bit (kin) of the two 32-key words; this lane's keys are kb4*16 + 4*g4 + r
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb4 = 0; kb4 < 4; ++kb4) {
          const uint32_t bits = w[qb][kb4 >> 1] >> ((kb4 & 1) * 16 + g4 * 4);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (kb4 * 16 + g4 * 4 + r >= rem || !((bits >> r) & 1u)) sacc[qb][kb4][r] = -INFINITY;
        }
    } else if (rem < kTile) {
      asm volatile("" ::: "memory");  // a real branch: taken on a split's last tile only
#pragma unroll
      for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (kb4 * 16 + g4 * 4 + r >= rem) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) sacc[qb][kb4][r] = -INFINITY;
          }
    }
    // ---- online softmax (base 2), lazy rescale
    bool need[2] = {false, false};
    float tmax[2], m_use[2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb4 = 0; kb4 < 4; ++kb4)
        mx = fmaxf(mx, fmaxf(fmaxf(sacc[qb][kb4][0], sacc[qb][kb4][1]), fmaxf(sacc[qb][kb4][2], sacc[qb][kb4][3])));
      mx = fmaxf(mx, xchg<16>(mx));
      mx = fmaxf(mx, xchg<32>(mx));
      tmax[qb] = mx * scale_log2;
      need[qb] = tmax[qb] > m_run[qb] + kTau;   // always true on the first unmasked tile
    }
    if (ballot(need[0] || need[1])) {
      // a real branch, taken rarely: left to itself the compiler runs this body on every
      // tile as selects (74 multiplies per tile)
      asm volatile("" ::: "memory");
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float m_new = need[qb] ? tmax[qb] : m_run[qb];
        const float alpha = m_run[qb] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[qb] - m_new);
        m_run[qb] = m_new;
        lacc[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < 8; ++db) oacc[qb][db] *= alpha;
      }
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) m_use[qb] = m_run[qb] == -INFINITY ? 0.f : m_run[qb];
    bf16x8 pb[2][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[qb][kb4][r], scale_log2, -m_use[qb]));
          pb[qb][kb4 / 2][(kb4 & 1) * 4 + r] = (bf16_t)p;
        }
    __builtin_amdgcn_sched_barrier(0);
    // ---- O^T += V^T . P^T  (V^T read transposed from the row-major tile).  The two
    // key rows a lane addresses (vrow, vrow + 16, plus 32 per key half) share one
    // swizzle, so the chunk slot is (2 db) ^ vsw_hi | vsw_lo.  Head-dim blocks go in
    // pairs: a pair's eight MFMAs alternate four accumulators, and the next pair's eight
    // fragment reads are issued while they run.
    auto vread = [&](int db, bf16x8 (&a)[2]) {
      const int slot = (((2 * db) ^ vhi) | vlo) << 4;
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const unsigned char* p = Vs + vb_ + kh * 32 * 256 + slot;
        const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
        const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 16 * 256));
        a[kh] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    };
    bf16x8 va[2][2][2];  // [buffer][db of the pair][kh]
    vread(0, va[0][0]);
    vread(1, va[0][1]);
    // sum_k P[k][q] for every query: the same contraction with V replaced by ones
    // (the sum is of the bf16 weights the numerator uses); these cover the first reads
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
        lacc[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[qb][kh], lacc[qb], 0, 0, 0);
#pragma unroll
    for (int pr = 0; pr < 4; ++pr) {
      if (pr + 1 < 4) {
        vread(2 * pr + 2, va[(pr + 1) & 1][0]);
        vread(2 * pr + 3, va[(pr + 1) & 1][1]);
      }
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            oacc[qb][2 * pr + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[pr & 1][j][kh], pb[qb][kh],
                                                                            oacc[qb][2 * pr + j], 0, 0, 0);
    }
    // order: the first pair's reads, the row sums, then per pair QB MFMAs per two
    // reads of the next pair (one and one for two blocks)
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 1);
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * QB, 1);
#pragma unroll
    for (int pr = 0; pr < 3; ++pr)
#pragma unroll
      for (int i = 0; i < 8 / (3 - QB); ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 3 - QB, 1);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      }
    __builtin_amdgcn_sched_group_barrier(0x008, 4 * QB, 1);
  };

  // ---- one tile from ring stage ST
  auto step = [&]<int ST>(int t) {
    // wait for this wave's loads of tile t: the only loads in flight (expcnt and
    // lgkmcnt left at their maxima), then an execution barrier only: every wave has
    // waited for its own loads, and the stage refilled next was read one barrier ago
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __builtin_amdgcn_s_barrier();
    // the tree split's mask words for this tile, issued ahead of the next tile's loads so
    // that waiting for them leaves those in flight.  The tile's 64 keys span words wi and
    // wi + 1; wi < W always (the tile starts below nn <= N), and when wi + 1 == W the
    // second word's keys all lie past N, masked by the tail test, so it re-reads word wi.
    uint32_t w[2][2];
    if (tree) {
      const uint32_t wi = (uint32_t)t * (kTile / 32);
      const uint32_t wj = min(wi + 1, (uint32_t)W - 1);
      w[0][0] = *(const uint32_t*)(mseq + (mrow0 + wi * 4));
      w[0][1] = *(const uint32_t*)(mseq + (mrow0 + wj * 4));
      w[1][0] = *(const uint32_t*)(mseq + (mrow1 + wi * 4));
      w[1][1] = *(const uint32_t*)(mseq + (mrow1 + wj * 4));
    }
    if (t + 1 < ntiles) issue.template operator()<ST ^ 1>(t + 1);
    if (live) math.template operator()<ST, 2>(t, w);
  };

  if (!solo) {
    // prologue: tile 0 in flight.  Tile t uses stage t % 2; the loop is unrolled by the
    // ring depth so every stage is a distinct object at compile time.
    if (0 < ntiles) issue.template operator()<0>(0);
    if (0 < ntiles) step.template operator()<0>(0);
    for (int t = 1; t < ntiles; t += kStages) {
      step.template operator()<1>(t);
      if (t + 1 < ntiles) step.template operator()<0>(t + 1);
    }
  } else {
    // Wave ST (0 or 1) takes tiles ST, ST + 2, ... through stage ST: it waits for its
    // own loads only, and refills the stage once its reads of it have returned.
    const uint32_t wz[2][2] = {{0u, 0u}, {0u, 0u}};
    auto stream = [&]<int ST, int QB>() {
      if (ST < ntiles) issue.template operator()<ST, 1>(ST);
      for (int t = ST; t < ntiles; t += 2) {
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): tile t is in the stage
        math.template operator()<ST, QB>(t, wz);
        if (t + 2 < ntiles) {
          __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): every read of the stage returned
          issue.template operator()<ST, 1>(t + 2);
        }
      }
    };
    if (wave == 0) {
      if (one_qb) stream.template operator()<0, 1>();
      else stream.template operator()<0, 2>();
    } else if (wave == 1) {
      if (one_qb) stream.template operator()<1, 1>();
      else stream.template operator()<1, 2>();
    }
    // wave 1 hands its (O, max, sum) to wave 0 through the ring, now idle: O as
    // [qb][db][lane] f32x4 in the K stages, (max, sum) as [qb][lane] in a V stage
    f32x4* xo = reinterpret_cast<f32x4*>(g_ring_k0);
    f32x2* xml = reinterpret_cast<f32x2*>(g_ring_v0);
    __syncthreads();
    if (wave == 1) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        if (qb == 1 && one_qb) break;
#pragma unroll
        for (int db = 0; db < 8; ++db) xo[(qb * 8 + db) * 64 + lane] = oacc[qb][db];
        xml[qb * 64 + lane] = f32x2{m_run[qb], lacc[qb][0]};
      }
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      if (qb == 1 && one_qb) break;
      const f32x2 o1 = xml[qb * 64 + lane];
      const float m0 = m_run[qb], m1 = o1[0];
      const float mm = fmaxf(m0, m1);
      // a stream that saw no tile holds max -inf, sum 0 and O = 0
      const float a0 = m0 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m0 - mm);
      const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
      m_run[qb] = mm;
      lacc[qb][0] = a0 * lacc[qb][0] + a1 * o1[1];
#pragma unroll
      for (int db = 0; db < 8; ++db) oacc[qb][db] = a0 * oacc[qb][db] + a1 * xo[(qb * 8 + db) * 64 + lane];
    }
  }

  // ---- partial results of this split
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float lt = lacc[qb][0];
    if (rowq[qb] < R) {
      const int64_t urow = (((int64_t)u.s * Hkv + u.g) * (nsplit + 1) + u.c) * rows_pad + rowq[qb];
      float* orow = opart + urow * D;
#pragma unroll
      for (int db = 0; db < 8; ++db)
        __builtin_nontemporal_store(oacc[qb][db], reinterpret_cast<f32x4*>(orow + db * 16 + g4 * 4));
      if (g4 == 0) __builtin_nontemporal_store(f32x2{m_run[qb], lt}, reinterpret_cast<f32x2*>(mlpart + urow));
    }
  }
}

// Blocks of 128 threads (D / 4 per row).  More, smaller blocks start sooner on a small
// grid (C1: 1.7 us less per attention call back to back than 256-thread blocks, 0.4%
// more rounds/s in the full round; C2 and C3 unchanged).
constexpr int kCombineThreads = 128;

// Merge the splits of each row: out = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c.
// The splits are read in batches of KB whose loads are all issued before any is
// used, and the batches are merged online (running max, rescaled sums), so a row
// costs one memory latency per KB splits.  The host picks KB >= the split count
// where it can, making the whole merge one latency.
template <typename OutT, int D, int KB>
__global__ void __launch_bounds__(kCombineThreads)
attn_combine(const float* __restrict__ opart, const float2* __restrict__ mlpart,
             Prefix pre, const int32_t* __restrict__ num_nodes, int S,
             int N, int Hq, int Hkv, int G, int rows_pad, int nsplit, int64_t chunk,
             bool has_cache, OutT* __restrict__ out, float* __restrict__ lse) {
  constexpr int TPR = D / 4;            // threads per row, 4 outputs each
  constexpr int RPB = kCombineThreads / TPR;  // rows per block
  const int64_t rid = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int dq = (threadIdx.x % TPR) * 4;
  if (rid >= (int64_t)S * N * Hq) return;
  const int h = (int)(rid % Hq);
  const int n = (int)((rid / Hq) % N);
  const int s = (int)(rid / ((int64_t)Hq * N));
  OutT* o = out + rid * D + dq;
  if (n >= num_nodes[s]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (OutT)0.f;
    if (lse && dq == 0) lse[rid] = -INFINITY;
    return;
  }
  const int g = h / G;
  const int row = n * G + (h % G);
  const int64_t P = has_cache ? pre.length(s) : 0;
  const int nvalid = P > 0 ? (int)min<int64_t>(nsplit, (P + chunk - 1) / chunk) : 0;
  const int64_t base = ((int64_t)s * Hkv + g) * (nsplit + 1);
  // the splits that hold keys: prefix splits 0 .. nvalid-1, then the tree split
  const int nused = nvalid + 1;
  auto split_of = [&](int i) { return i < nvalid ? i : nsplit; };
  float M = -INFINITY;
  float l = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int i0 = 0; i0 < nused; i0 += KB) {
    float2 ml[KB];
    f32x4 v[KB];
#pragma unroll
    for (int b = 0; b < KB; ++b) {
      const bool ok = i0 + b < nused;
      const int64_t ur = (base + split_of(ok ? i0 + b : 0)) * rows_pad + row;
      ml[b] = ok ? mlpart[ur] : make_float2(-INFINITY, 0.f);
      v[b] = ok ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(opart + ur * D + dq))
                : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float bm = M;
#pragma unroll
    for (int b = 0; b < KB; ++b) bm = fmaxf(bm, ml[b].x);
    if (bm == -INFINITY) continue;  // nothing visible yet (cannot happen: the root sees itself)
    if (M != -INFINITY && M != bm) {
      const float r = __builtin_amdgcn_exp2f(M - bm);
      l *= r;
      acc *= r;
    }
    M = bm;
#pragma unroll
    for (int b = 0; b < KB; ++b) {
      const float w = (ml[b].x == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ml[b].x - M);
      l += w * ml[b].y;
      acc += w * v[b];
    }
  }
  const float inv = 1.f / l;
  o[0] = (OutT)(acc[0] * inv);
  o[1] = (OutT)(acc[1] * inv);
  o[2] = (OutT)(acc[2] * inv);
  o[3] = (OutT)(acc[3] * inv);
  if (lse && dq == 0) lse[rid] = (M + __log2f(l)) * kLn2;
}

// ---------------------------------------------------------------- fp32 path
template <int D>
__global__ void __launch_bounds__(64)
attn_f32(const float* __restrict__ q, const float* __restrict__ kc, const float* __restrict__ vc,
         Prefix pre, const float* __restrict__ kt,
         const float* __restrict__ vt, const uint32_t* __restrict__ mask,
         const int32_t* __restrict__ num_nodes, int N, int Hq, int Hkv, int W, float scale,
         float* __restrict__ out, float* __restrict__ lse) {
  constexpr int DPL = (D + 63) / 64;  // head-dim entries per lane
  __shared__ float qs[D];
  __shared__ int vis[64];
  const int64_t rid = blockIdx.x;
  const int lane = threadIdx.x;
  const int h = (int)(rid % Hq);
  const int n = (int)((rid / Hq) % N);
  const int s = (int)(rid / ((int64_t)Hq * N));
  float* o = out + rid * D;
  if (n >= num_nodes[s]) {
    for (int d = lane; d < D; d += 64) o[d] = 0.f;
    if (lse && lane == 0) lse[rid] = -INFINITY;
    return;
  }
  const int g = h / (Hq / Hkv);
  for (int d = lane; d < D; d += 64) qs[d] = q[rid * D + d];
  __syncthreads();
  const int64_t p0 = pre.start(s);
  const int64_t P = kc ? pre.length(s) : 0;
  float m = -INFINITY, l = 0.f;
  float acc[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc[i] = 0.f;

  // one tile of up to 64 keys, key j of the tile at kbase + idx(j) * stride
  auto tile = [&](const float* kbase, const float* vbase, int cnt, auto idx) {
    float sc = -INFINITY;
    if (lane < cnt) {
      const float* kr = kbase + (int64_t)idx(lane) * Hkv * D;
      float dot = 0.f;
      for (int d = 0; d < D; ++d) dot += qs[d] * kr[d];
      sc = dot * scale;
    }
    const float mt = wave_max(sc);
    const float mn = fmaxf(m, mt);
    const float alpha = __expf(m - mn);
    const float p = lane < cnt ? __expf(sc - mn) : 0.f;
    float ps = p;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ps += __shfl_xor(ps, off);
    l = l * alpha + ps;
#pragma unroll
    for (int i = 0; i < DPL; ++i) acc[i] *= alpha;
    for (int j = 0; j < cnt; ++j) {
      const float pj = __shfl(p, j);
      const float* vr = vbase + (int64_t)idx(j) * Hkv * D;
#pragma unroll
      for (int i = 0; i < DPL; ++i) {
        const int d = lane + 64 * i;
        if (d < D) acc[i] += pj * vr[d];
      }
    }
    m = mn;
  };
  const float* kpre = kc + (p0 * Hkv + g) * D;
  const float* vpre = vc + (p0 * Hkv + g) * D;
  for (int64_t t0 = 0; t0 < P; t0 += 64) {
    const int cnt = (int)min<int64_t>(64, P - t0);
    tile(kpre + t0 * Hkv * D, vpre + t0 * Hkv * D, cnt, [](int j) { return j; });
  }
  // visible tree nodes, 64 at a time
  const uint32_t* mrow = mask + ((int64_t)s * N + n) * W;
  const float* ktr = kt + ((int64_t)s * N * Hkv + g) * D;
  const float* vtr = vt + ((int64_t)s * N * Hkv + g) * D;
  int cnt = 0;
  for (int j0 = 0; j0 < N; j0 += 64) {
    const int j = j0 + lane;
    const bool on = j < N && ((mrow[j >> 5] >> (j & 31)) & 1u);
    const unsigned long long b = ballot(on);
    const int before = __popcll(b & ((1ull << lane) - 1ull));
    const int total = __popcll(b);
    // flush when the list would overflow 64
    if (cnt + total > 64) {
      __syncthreads();
      tile(ktr, vtr, cnt, [&](int x) { return vis[x]; });
      __syncthreads();
      cnt = 0;
    }
    if (on) vis[cnt + before] = j;
    cnt += total;
  }
  __syncthreads();
  if (cnt > 0) tile(ktr, vtr, cnt, [&](int x) { return vis[x]; });
  const float inv = 1.f / l;
#pragma unroll
  for (int i = 0; i < DPL; ++i) {
    const int d = lane + 64 * i;
    if (d < D) o[d] = acc[i] * inv;
  }
  if (lse && lane == 0) lse[rid] = m + logf(l);
}

template <int D, int NW>
hipError_t launch_partial(const AttnPlan& p, const void* q, const void* kc, const void* vc,
                          Prefix cu, const void* kt, const void* vt, const uint32_t* mask,
                          const int32_t* nn, int S, int N, int Hq, int Hkv, int W, float scale,
                          float* opart, float2* ml, hipStream_t st, hipEvent_t ev0,
                          hipEvent_t ev1) {
  const int units = S * Hkv * (p.nsplit + 1);
  const int blocks = (int)(ceil_div(units, 8) * 8 * p.row_groups);
  hipExtLaunchKernelGGL((attn_partial_bf16<D, NW>), dim3(blocks), dim3(NW * 64), Lds<D>::bytes,
                        st, ev0, ev1, 0, (const bf16_t*)q, (const bf16_t*)kc, (const bf16_t*)vc,
                        cu, (const bf16_t*)kt, (const bf16_t*)vt, mask, nn, N, Hq, Hkv, p.G, p.R,
                        W, p.rows_pad, p.nsplit, p.chunk, units, p.row_groups, scale * kLog2e,
                        opart, ml);
  return hipGetLastError();
}

template <int NW>
hipError_t launch_d128_nw(const AttnPlan& p, const void* q, const void* kc, const void* vc,
                          Prefix cu, const void* kt, const void* vt, const uint32_t* mask,
                          const int32_t* nn, int S, int N, int Hq, int Hkv, int W, float scale,
                          float* opart, float2* ml, hipStream_t st, hipEvent_t ev0,
                          hipEvent_t ev1) {
  const int units = S * Hkv * (p.nsplit + 1);
  const int blocks = (int)(ceil_div(units, 8) * 8 * p.row_groups);
  hipExtLaunchKernelGGL((attn_d128<NW>), dim3(blocks), dim3(NW * 64), 0, st, ev0, ev1, 0,
                        (const bf16_t*)q, (const bf16_t*)kc, (const bf16_t*)vc, cu,
                        (const bf16_t*)kt, (const bf16_t*)vt, mask, nn, N, Hq, Hkv, p.G, p.R, W,
                        p.rows_pad, p.nsplit, p.chunk, units, p.row_groups, scale * kLog2e, opart,
                        ml);
  return hipGetLastError();
}

hipError_t launch_d128(const AttnPlan& p, const void* q, const void* kc, const void* vc,
                       Prefix cu, const void* kt, const void* vt, const uint32_t* mask,
                       const int32_t* nn, int S, int N, int Hq, int Hkv, int W, float scale,
                       float* opart, float2* ml, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
#define DDT_NW(X)                                                                            \
  case X:                                                                                    \
    return launch_d128_nw<X>(p, q, kc, vc, cu, kt, vt, mask, nn, S, N, Hq, Hkv, W, scale,   \
                             opart, ml, st, ev0, ev1);
  switch (p.waves) {
    DDT_NW(1) DDT_NW(2) DDT_NW(3) DDT_NW(4) DDT_NW(5) DDT_NW(6) DDT_NW(7) DDT_NW(8)
    default:
      return hipErrorInvalidValue;
  }
#undef DDT_NW
}

template <int D>
hipError_t launch_partial_d(const AttnPlan& p, const void* q, const void* kc, const void* vc,
                            Prefix cu, const void* kt, const void* vt, const uint32_t* mask,
                            const int32_t* nn, int S, int N, int Hq, int Hkv, int W, float scale,
                            float* opart, float2* ml, hipStream_t st, hipEvent_t ev0,
                            hipEvent_t ev1) {
#define DDT_NW(X)                                                                                \
  case X:                                                                                        \
    return launch_partial<D, X>(p, q, kc, vc, cu, kt, vt, mask, nn, S, N, Hq, Hkv, W, scale, \
                                opart, ml, st, ev0, ev1);
  switch (p.waves) {
    DDT_NW(1) DDT_NW(2) DDT_NW(3) DDT_NW(4) DDT_NW(5) DDT_NW(6) DDT_NW(7) DDT_NW(8)
    default:
      return hipErrorInvalidValue;
  }
#undef DDT_NW
}

}  // namespace

AttnPlan attn_plan(int S, int B, int Hq, int Hkv, int D, int dtype, int64_t max_prefix) {
  AttnPlan p{};
  const int N = B + 1;
  p.dtype = dtype;
  p.D = D;
  p.G = Hq / Hkv;
  p.R = p.G * N;
  if (dtype != DDT_BF16) {
    p.waves = 1;
    p.row_groups = 1;
    p.rows_pad = 0;
    p.nsplit = 0;
    p.chunk = 0;
    p.ws_bytes = 0;
    return p;
  }
  if (D == 128) {
    // attn_d128, 32 rows per wave.  Wide groups (up to 8 waves, one workgroup per CU)
    // when the whole grid fits on the CUs at once, which is the latency-bound case;
    // otherwise groups of up to 4 waves, two workgroups per CU.
    const int waves = (int)ceil_div(p.R, 32);
    const int rg_wide = (int)ceil_div(waves, 8);
    const int64_t units_wide = (int64_t)S * Hkv * rg_wide;
    const int64_t maxp = std::max<int64_t>(max_prefix, 0);
    const int64_t want = std::max<int64_t>(1, ceil_div(2 * (int64_t)cu_count(), units_wide));
    const int64_t chunk_w = std::max<int64_t>(
        (int64_t)align_up((size_t)std::max<int64_t>(1, ceil_div(maxp, want)), kTile), kTile);
    const int64_t splits_w = std::max<int64_t>(1, ceil_div(maxp, chunk_w)) + 1;
    if (units_wide * splits_w <= cu_count()) {
      p.row_groups = rg_wide;
      p.waves = (int)ceil_div(waves, rg_wide);
    } else {
      p.waves = waves < 4 ? waves : 4;
      p.row_groups = (int)ceil_div(waves, p.waves);
    }
  } else {
    const int tiles = (int)ceil_div(p.R, 32);
    p.row_groups = (int)ceil_div(tiles, 8);
    p.waves = (int)ceil_div(tiles, p.row_groups);
  }
  p.rows_pad = p.row_groups * p.waves * 32;
  // prefix splits: about three (sequence, KV head, row group, split) units per CU
  // (measured best on C2, C3 B >= 256 and C4 against one, two and four), and no split
  // above 12K keys so that unequal prefix lengths still spread evenly.  The cap decides
  // only when the units alone exceed three per CU (32 sequences of 16K-32K keys): there
  // the splits are dealt to the resident workgroup slots in rounds, and 12K keys packed
  // those rounds best (paired runs at that shape, main kernel plus merge: 4K +1%, 8K
  // and 10K -1 to -2%, 12K -3.7%, 14K 0, 32K +8%, against 16K).  With few
  // (sequence, KV head, row group) units, up to a quarter of the CUs, three per CU cuts
  // each unit into many splits of two to four tiles, whose partials outweigh the keys
  // they cover; one per CU is then better (paired runs: C3 B = 16 to 128, +6-10%
  // rounds/s).  Since the short remainder groups stream on their own, units with
  // fewer than 16 row groups pack better at two per CU (paired, against three: C2, 3
  // groups, +2.1% rounds/s; C3 B = 256, 9 groups, +1.0%), while C3 B = 512 (17 groups)
  // keeps three (two: -1.6%); the boundary between 9 and 17 is set by these runs alone.
  const int64_t units_base = (int64_t)S * Hkv * p.row_groups;
  const int64_t per_cu = D != 128 ? 2 : units_base * 4 <= cu_count() ? 1 : p.row_groups < 16 ? 2 : 3;
  const int64_t target = per_cu * (int64_t)cu_count();
  const int64_t maxp = std::max<int64_t>(max_prefix, 0);
  const int64_t want = std::max<int64_t>(1, ceil_div(target, units_base));
  int64_t chunk = (int64_t)align_up((size_t)std::max<int64_t>(1, ceil_div(maxp, want)), kTile);
  chunk = std::min<int64_t>(std::max<int64_t>(chunk, kTile), 12288);
  p.chunk = chunk;
  p.nsplit = (int)std::max<int64_t>(1, ceil_div(maxp, chunk));
  const size_t rows = (size_t)S * Hkv * (p.nsplit + 1) * p.rows_pad;
  p.ws_bytes = align_up(rows * D * sizeof(float), 256) + align_up(rows * sizeof(float2), 256);
  return p;
}

hipError_t launch_tree_attention(const void* q, const void* kc, const void* vc,
                                 Prefix pre, const void* kt, const void* vt,
                                 const uint32_t* mask, const int32_t* num_nodes, int S, int B,
                                 int Hq, int Hkv, int D, float scale, void* out, float* lse,
                                 void* ws, const AttnPlan& p, hipStream_t st) {
  const int N = B + 1;
  const int W = (N + 31) / 32;
  if (p.dtype == DDT_F32) {
    const int64_t rows = (int64_t)S * N * Hq;
    hipEvent_t ev0 = nullptr, ev1 = nullptr;
    if (!prof_events(&ev0, &ev1, nullptr)) ev0 = ev1 = nullptr;
#define DDT_F32_D(DD)                                                                          \
  case DD:                                                                                     \
    hipExtLaunchKernelGGL(attn_f32<DD>, dim3((unsigned)rows), dim3(64), 0, st, ev0, ev1, 0,    \
                          (const float*)q, (const float*)kc, (const float*)vc, pre,            \
                          (const float*)kt, (const float*)vt, mask, num_nodes, N, Hq, Hkv, W,  \
                          scale, (float*)out, lse);                                            \
    return hipGetLastError();
    switch (D) {
      DDT_F32_D(32) DDT_F32_D(64) DDT_F32_D(128)
      default:
        return hipErrorInvalidValue;
    }
#undef DDT_F32_D
  }
  const size_t rows = (size_t)S * Hkv * (p.nsplit + 1) * p.rows_pad;
  float* opart = static_cast<float*>(ws);
  float2* ml = reinterpret_cast<float2*>(static_cast<char*>(ws) + align_up(rows * D * sizeof(float), 256));
  hipError_t e;
  hipEvent_t ev0 = nullptr, ev1 = nullptr, ev2 = nullptr;
  if (!prof_events(&ev0, &ev1, &ev2)) ev0 = ev1 = ev2 = nullptr;
  switch (D) {
    case 32: e = launch_partial_d<32>(p, q, kc, vc, pre, kt, vt, mask, num_nodes, S, N, Hq, Hkv, W, scale, opart, ml, st, ev0, ev1); break;
    case 64: e = launch_partial_d<64>(p, q, kc, vc, pre, kt, vt, mask, num_nodes, S, N, Hq, Hkv, W, scale, opart, ml, st, ev0, ev1); break;
    case 128: e = launch_d128(p, q, kc, vc, pre, kt, vt, mask, num_nodes, S, N, Hq, Hkv, W, scale, opart, ml, st, ev0, ev1); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  const int64_t total = (int64_t)S * N * Hq;
  const int rpb = kCombineThreads / (D / 4);
  const unsigned blocks = (unsigned)ceil_div(total, rpb);
  // splits per batch: enough for every split of a row when that fits in registers
  const int nused = p.nsplit + 1;
  const int kb = nused <= 2 ? 2 : nused <= 4 ? 4 : nused <= 8 ? 8 : nused <= 16 ? 16 : 32;
#define DDT_COMB_KB(DD, KK)                                                                     \
  hipExtLaunchKernelGGL((attn_combine<bf16_t, DD, KK>), dim3(blocks), dim3(kCombineThreads), 0, \
                        st, nullptr, ev2, 0, opart, ml, pre, num_nodes, S, N, Hq, Hkv,          \
                        p.G, p.rows_pad, p.nsplit, p.chunk, kc != nullptr, (bf16_t*)out, lse)
#define DDT_COMB(DD)                                     \
  case DD:                                               \
    switch (kb) {                                        \
      case 2: DDT_COMB_KB(DD, 2); break;                 \
      case 4: DDT_COMB_KB(DD, 4); break;                 \
      case 8: DDT_COMB_KB(DD, 8); break;                 \
      case 16: DDT_COMB_KB(DD, 16); break;               \
      default: DDT_COMB_KB(DD, 32); break;               \
    }                                                    \
    break;
  switch (D) {
    DDT_COMB(32) DDT_COMB(64) DDT_COMB(128)
    default:
      return hipErrorInvalidValue;
  }
#undef DDT_COMB
#undef DDT_COMB_KB
  return hipGetLastError();
}

}  // namespace ddt
