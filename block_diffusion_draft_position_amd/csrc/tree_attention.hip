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
//   Per wave and 32-key half-tile, with the MFMA v_mfma_f32_32x32x16_bf16:
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
// fp32 path: one wave per query row over all of its keys (no splits), VALU only.
#include <math.h>

#include "ddt_internal.h"

namespace ddt {
namespace {

typedef __bf16 bf16_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
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
// and share that XCD's L2 for the unit's K/V.
__device__ __forceinline__ bool decode_block(int Hkv, int nsplit_tot, int row_groups, int units,
                                             Unit& u) {
  const int blk = blockIdx.x;
  const int x8 = blk & 7;
  const int rest = blk >> 3;
  u.rg = rest % row_groups;
  const int un = (rest / row_groups) * 8 + x8;
  if (un >= units) return false;
  u.c = un % nsplit_tot;
  const int sg = un / nsplit_tot;
  u.g = sg % Hkv;
  u.s = sg / Hkv;
  return true;
}

template <int D, int NW>
__global__ void __launch_bounds__(NW * 64)
attn_partial_bf16(const bf16_t* __restrict__ q, const bf16_t* __restrict__ kc,
                  const bf16_t* __restrict__ vc, const int64_t* __restrict__ cu_prefix,
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
  const int64_t p0 = cu_prefix[u.s];
  const int64_t P = kc ? cu_prefix[u.s + 1] - p0 : 0;
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
        *reinterpret_cast<float4*>(orow + d) =
            make_float4(oacc[db][4 * qq], oacc[db][4 * qq + 1], oacc[db][4 * qq + 2], oacc[db][4 * qq + 3]);
      }
    }
    if (h2 == 0) mlpart[urow] = make_float2(m_run, l_tot);
  }
}

// Merge the splits of each row: out = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c.
template <typename OutT, int D>
__global__ void __launch_bounds__(256)
attn_combine(const float* __restrict__ opart, const float2* __restrict__ mlpart,
             const int64_t* __restrict__ cu_prefix, const int32_t* __restrict__ num_nodes, int S,
             int N, int Hq, int Hkv, int G, int rows_pad, int nsplit, int64_t chunk,
             bool has_cache, OutT* __restrict__ out, float* __restrict__ lse) {
  constexpr int TPR = D / 4;            // threads per row, 4 outputs each
  constexpr int RPB = 256 / TPR;        // rows per block
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
  const int64_t P = has_cache ? cu_prefix[s + 1] - cu_prefix[s] : 0;
  const int nvalid = P > 0 ? (int)min<int64_t>(nsplit, (P + chunk - 1) / chunk) : 0;
  const int64_t base = ((int64_t)s * Hkv + g) * (nsplit + 1);
  float M = mlpart[(base + nsplit) * rows_pad + row].x;
  for (int c = 0; c < nvalid; ++c) M = fmaxf(M, mlpart[(base + c) * rows_pad + row].x);
  float l = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int c = 0; c <= nsplit; ++c) {
    if (c < nsplit && c >= nvalid) continue;
    const int64_t ur = (base + c) * rows_pad + row;
    const float2 ml = mlpart[ur];
    const float w = (ml.x == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ml.x - M);
    l += w * ml.y;
    const float4 v = *reinterpret_cast<const float4*>(opart + ur * D + dq);
    acc.x += w * v.x;
    acc.y += w * v.y;
    acc.z += w * v.z;
    acc.w += w * v.w;
  }
  const float inv = 1.f / l;
  o[0] = (OutT)(acc.x * inv);
  o[1] = (OutT)(acc.y * inv);
  o[2] = (OutT)(acc.z * inv);
  o[3] = (OutT)(acc.w * inv);
  if (lse && dq == 0) lse[rid] = (M + __log2f(l)) * kLn2;
}

// ---------------------------------------------------------------- fp32 path
template <int D>
__global__ void __launch_bounds__(64)
attn_f32(const float* __restrict__ q, const float* __restrict__ kc, const float* __restrict__ vc,
         const int64_t* __restrict__ cu_prefix, const float* __restrict__ kt,
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
  const int64_t p0 = cu_prefix[s];
  const int64_t P = kc ? cu_prefix[s + 1] - p0 : 0;
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
                          const int64_t* cu, const void* kt, const void* vt, const uint32_t* mask,
                          const int32_t* nn, int S, int N, int Hq, int Hkv, int W, float scale,
                          float* opart, float2* ml, hipStream_t st) {
  const int units = S * Hkv * (p.nsplit + 1);
  const int blocks = (int)(ceil_div(units, 8) * 8 * p.row_groups);
  hipLaunchKernelGGL((attn_partial_bf16<D, NW>), dim3(blocks), dim3(NW * 64), Lds<D>::bytes, st,
                     (const bf16_t*)q, (const bf16_t*)kc, (const bf16_t*)vc, cu,
                     (const bf16_t*)kt, (const bf16_t*)vt, mask, nn, N, Hq, Hkv, p.G, p.R, W,
                     p.rows_pad, p.nsplit, p.chunk, units, p.row_groups, scale * kLog2e, opart,
                     ml);
  return hipGetLastError();
}

template <int D>
hipError_t launch_partial_d(const AttnPlan& p, const void* q, const void* kc, const void* vc,
                            const int64_t* cu, const void* kt, const void* vt, const uint32_t* mask,
                            const int32_t* nn, int S, int N, int Hq, int Hkv, int W, float scale,
                            float* opart, float2* ml, hipStream_t st) {
#define DDT_NW(X)                                                                                \
  case X:                                                                                        \
    return launch_partial<D, X>(p, q, kc, vc, cu, kt, vt, mask, nn, S, N, Hq, Hkv, W, scale, \
                                opart, ml, st);
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
  const int tiles = (int)ceil_div(p.R, 32);
  p.row_groups = (int)ceil_div(tiles, 8);
  p.waves = (int)ceil_div(tiles, p.row_groups);
  p.rows_pad = p.row_groups * p.waves * 32;
  const int64_t units_base = (int64_t)S * Hkv * p.row_groups;
  const int64_t target = 2 * (int64_t)cu_count();
  const int64_t maxp = std::max<int64_t>(max_prefix, 0);
  const int64_t want = std::max<int64_t>(1, ceil_div(target, units_base));
  int64_t chunk = (int64_t)align_up((size_t)std::max<int64_t>(1, ceil_div(maxp, want)), kTile);
  chunk = std::max<int64_t>(chunk, 2 * kTile);
  p.chunk = chunk;
  p.nsplit = (int)std::max<int64_t>(1, ceil_div(maxp, chunk));
  const size_t rows = (size_t)S * Hkv * (p.nsplit + 1) * p.rows_pad;
  p.ws_bytes = align_up(rows * D * sizeof(float), 256) + align_up(rows * sizeof(float2), 256);
  return p;
}

hipError_t launch_tree_attention(const void* q, const void* kc, const void* vc,
                                 const int64_t* cu_prefix, const void* kt, const void* vt,
                                 const uint32_t* mask, const int32_t* num_nodes, int S, int B,
                                 int Hq, int Hkv, int D, float scale, void* out, float* lse,
                                 void* ws, const AttnPlan& p, hipStream_t st) {
  const int N = B + 1;
  const int W = (N + 31) / 32;
  if (p.dtype == DDT_F32) {
    const int64_t rows = (int64_t)S * N * Hq;
#define DDT_F32_D(DD)                                                                          \
  case DD:                                                                                     \
    hipLaunchKernelGGL(attn_f32<DD>, dim3((unsigned)rows), dim3(64), 0, st, (const float*)q,   \
                       (const float*)kc, (const float*)vc, cu_prefix, (const float*)kt,        \
                       (const float*)vt, mask, num_nodes, N, Hq, Hkv, W, scale, (float*)out, lse); \
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
  const hipEvent_t stop = prof_begin(st);
  switch (D) {
    case 32: e = launch_partial_d<32>(p, q, kc, vc, cu_prefix, kt, vt, mask, num_nodes, S, N, Hq, Hkv, W, scale, opart, ml, st); break;
    case 64: e = launch_partial_d<64>(p, q, kc, vc, cu_prefix, kt, vt, mask, num_nodes, S, N, Hq, Hkv, W, scale, opart, ml, st); break;
    case 128: e = launch_partial_d<128>(p, q, kc, vc, cu_prefix, kt, vt, mask, num_nodes, S, N, Hq, Hkv, W, scale, opart, ml, st); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  if (stop) {
    e = prof_record(stop, st);
    if (e != hipSuccess) return e;
  }
  const int64_t total = (int64_t)S * N * Hq;
  const int rpb = 256 / (D / 4);
  const unsigned blocks = (unsigned)ceil_div(total, rpb);
#define DDT_COMB(DD)                                                                             \
  case DD:                                                                                       \
    hipLaunchKernelGGL((attn_combine<bf16_t, DD>), dim3(blocks), dim3(256), 0, st, opart, ml,    \
                       cu_prefix, num_nodes, S, N, Hq, Hkv, p.G, p.rows_pad, p.nsplit, p.chunk, \
                       kc != nullptr, (bf16_t*)out, lse);                                        \
    break;
  switch (D) {
    DDT_COMB(32) DDT_COMB(64) DDT_COMB(128)
    default:
      return hipErrorInvalidValue;
  }
#undef DDT_COMB
  return hipGetLastError();
}

}  // namespace ddt
