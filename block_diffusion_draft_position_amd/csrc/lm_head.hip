// Fused verifier epilogue: the target's LM head and greedy token at every tree node,
// without storing the logits (DDTree page "策展 · X (Twitter)": the target scores the
// tree in one forward, 運作流程 step 3, and the walk follows its greedy choice, step 4;
// a node's logits are its final hidden state times the output-embedding weight).
//
//   node_tok[m] = argmax_v fp32(h_m . w_v), equal values to the smaller v
//
// for the M = S * N hidden rows h_m [d] and vocabulary rows w_v [d], bf16, fp32
// accumulation.  Then the tree walk driven by those tokens.
//
// lm_head_tiles<VT, MT, NWV, NWM>: one workgroup per VT x MT tile of the logits
// (vocabulary x hidden rows), K = d in steps of 64.
//   * Tile shape by the number of hidden rows M: 256 x 256 with eight waves (each 128
//     vocabulary x 64 hidden rows, two waves per SIMD) above 128 rows; 256 x 128 with
//     four waves above 64; narrower below.  Each K-step brings (VT + MT) rows of 128
//     bytes into LDS for VT * MT * 128 flops: the 256 x 128 tile needs 48 bytes per
//     clock per CU from L2 to keep the MFMAs busy, about what the L2 delivers, and the
//     256 x 256 tile 32 (measured against the 256 x 128 tile: 32 x 65 rows 4.68 ->
//     3.75 ms; 520 and 513 rows -13 to -14%; 129 rows -23%).
//   * In the last row tile a wave's 32-row blocks with no live hidden row are neither
//     read nor multiplied (a separate copy of the K loop, so that full tiles carry no
//     test): with 2080 rows, the ninth 256-row tile holds 32.
//   * W and H tiles go global -> LDS by buffer_load_dwordx4 ... lds (no registers in
//     between) into a ring of NS stages (2 for the 256 x 256 tile: 128 KB; 3 for the
//     256 x 128 tile: 144 KB; one workgroup per CU; 2 for the narrow tiles).  An LDS
//     row is one tile row's 64 K-values, 128 bytes in eight 16-byte slots; chunk c of
//     row r sits in slot c ^ ((r >> 1) & 7), so that the 16 rows a 16-lane group reads
//     in one fragment load fall in 16 distinct 16-byte bank groups (measured: no bank
//     conflicts).
//   * One barrier per K-step, placed before the step's last substep: by then each wave
//     holds that substep's fragments in registers, so the stage can be refilled, and
//     having waited for its own loads of the next step, the next step's first
//     fragments are read while the last substep's MFMAs run.  Within a step each
//     substep's MFMAs are interleaved with the next substep's fragment reads.
//   * Logits^T tiles on v_mfma_f32_32x32x16_bf16 with the vocabulary rows as the A
//     operand and the hidden rows as B: a lane's accumulators then hold one hidden row
//     (its column) against 16 vocabulary rows, so the arg-max is in-lane first.
//   * Epilogue: each lane's best (value, id) over its vocabulary rows, then the lane
//     pair that shares the column, then the waves that share it (through LDS); one
//     (value, id) partial per (hidden row, vocabulary tile).
// lm_head_reduce: one wave per hidden row over its partials.
// tree_walk_tokens_kernel: one wave per sequence.
#include <hip/hip_ext.h>

#include "ddt_internal.h"

namespace ddt {
namespace {

typedef __bf16 bf16_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kKStep = 64;                       // K-values per ring stage
constexpr int kRowBytes = kKStep * 2;            // one tile row in LDS
constexpr int kRsrcWord3 = 0x00020000;           // gfx9-family raw buffer: 32-bit data format

struct Partial {
  float v;
  int i;
};

__device__ __forceinline__ int64_t rfl64(int64_t v) {
  const int lo32 = __builtin_amdgcn_readfirstlane((int)(v & 0xffffffff));
  const int hi32 = __builtin_amdgcn_readfirstlane((int)(v >> 32));
  return (int64_t)(((uint64_t)(uint32_t)hi32 << 32) | (uint32_t)lo32);
}

template <int VT, int MT, int NWV, int NWM, int NS>
struct LmCfg {
  static constexpr int NW = NWV * NWM;
  static constexpr int VW = VT / NWV;            // vocabulary rows per wave
  static constexpr int MW = MT / NWM;            // hidden rows per wave
  static constexpr int VB = VW / 32;             // 32-row MFMA blocks
  static constexpr int MB = MW / 32;
  static constexpr int STAGE = (VT + MT) * kRowBytes;
  static constexpr int LDS = NS * STAGE;
  static constexpr int NINST = (VT + MT) / 8;    // 1 KB loads per stage (8 rows each)
  static constexpr int PER_WAVE = NINST / NW;
  static_assert(VW % 32 == 0 && MW % 32 == 0, "32-row blocks");
  static_assert(NINST % NW == 0, "loads deal evenly to the waves");
  static_assert(NWV * MT * (int)sizeof(Partial) <= LDS, "epilogue fits the ring");
  static_assert(NS == 2 || NS == 3, "ring stages");
  static_assert(PER_WAVE < 64, "vmcnt range");
};

template <int VT, int MT, int NWV, int NWM, int NS>
__global__ void __launch_bounds__(NWV * NWM * 64, (NS * (VT + MT) * kRowBytes <= 81920 ? 2 : 1))
lm_head_tiles(const bf16_t* __restrict__ H, const bf16_t* __restrict__ Wt, int M, int V, int d,
              int nvt, int nmt, int per_xcd, Partial* __restrict__ partial) {
  using C = LmCfg<VT, MT, NWV, NWM, NS>;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[C::LDS];

  // tiles are dealt to the eight XCDs (workgroup i runs on XCD i % 8) in contiguous
  // runs, vocabulary tile major: the row tiles of one vocabulary tile share an L2
  const int bid = blockIdx.x;
  const int t = (bid & 7) * per_xcd + (bid >> 3);
  if (t >= nvt * nmt) return;
  const int vt = t / nmt, mt = t % nmt;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64;
  const int l32 = lane % 32, h2 = lane / 32;
  const int wv = wave % NWV, wm = wave / NWV;
  const int v0 = vt * VT, m0 = mt * MT;
  const int vrows = __builtin_amdgcn_readfirstlane(min(VT, V - v0));
  const int mrows = __builtin_amdgcn_readfirstlane(min(MT, M - m0));
  const bool full = vrows == VT && mrows == MT;
  const uint32_t rowb = (uint32_t)d * 2;
  const int nk = d / kKStep;

  // buffer resources at the tile's first W row and first H row (uniform bases)
  const unsigned char* wb = (const unsigned char*)rfl64((int64_t)(Wt + (int64_t)v0 * d));
  const unsigned char* hb = (const unsigned char*)rfl64((int64_t)(H + (int64_t)m0 * d));
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void*)wb, (short)0, -1, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc((void*)hb, (short)0, -1, kRsrcWord3);

  // A load instruction q covers 8 tile rows r0 .. r0 + 7 (q < VT/8: W rows 8q; else H
  // rows 8(q - VT/8)); lane l writes LDS row r0 + l/8, slot l % 8, so it fetches
  // chunk (l % 8) ^ (((r0 + l/8) >> 1) & 7) = (l % 8) ^ ((l/8) >> 1) ^ (r0 & 8 ? 4 : 0).
  // In a full tile that is one lane offset XOR a uniform constant, the row block in the
  // scalar offset.
  const uint32_t lane_base = (uint32_t)(lane / 8) * rowb + (uint32_t)(((lane % 8) ^ ((lane / 8) >> 1)) * 16);
  auto issue = [&]<int ST>(int s) {
    const uint32_t k0b = (uint32_t)__builtin_amdgcn_readfirstlane(s) * (kKStep * 2);
    if (full) {
#pragma unroll
      for (int j = 0; j < C::PER_WAVE; ++j) {
        const int q = wave + j * C::NW;
        const bool isH = q >= VT / 8;
        const int r0 = isH ? 8 * (q - VT / 8) : 8 * q;
        unsigned char* dst = smem + ST * C::STAGE + (isH ? VT * kRowBytes : 0) + r0 * kRowBytes;
        const uint32_t x = (r0 & 8) ? 64u : 0u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(isH ? rh : rw, (lds_void*)dst, 16, lane_base ^ x,
                                                 (uint32_t)r0 * rowb + k0b, 0, 0);
      }
    } else {
      // a tile at the vocabulary or row edge: rows past the edge re-read the last row
      // (never selected: their values equal the last row's at larger ids, and the
      // epilogue skips them besides)
      asm volatile("" ::: "memory");
      int l8 = lane / 8, l7 = lane % 8;
      asm volatile("" : "+v"(l8), "+v"(l7));
#pragma unroll
      for (int j = 0; j < C::PER_WAVE; ++j) {
        const int q = wave + j * C::NW;
        const bool isH = q >= VT / 8;
        const int r0 = isH ? 8 * (q - VT / 8) : 8 * q;
        const int rows = isH ? mrows : vrows;
        unsigned char* dst = smem + ST * C::STAGE + (isH ? VT * kRowBytes : 0) + r0 * kRowBytes;
        const int r = r0 + l8;
        const uint32_t off = (uint32_t)min(r, rows - 1) * rowb + (uint32_t)((l7 ^ ((r >> 1) & 7)) * 16);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(isH ? rh : rw, (lds_void*)dst, 16, off, k0b, 0, 0);
      }
    }
  };

  f32x16 acc[C::VB][C::MB];
#pragma unroll
  for (int vb = 0; vb < C::VB; ++vb)
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) acc[vb][mb] = f32x16{};

  // fragment reads: lane l reads row (block base + l % 32), K-chunk 2 ks + h2, whose
  // slot is (2 ks + h2) ^ ((l % 32 >> 1) & 7); the block bases are multiples of 32
  const int frag_base = l32 * kRowBytes;
  const int fsw = (l32 >> 1) & 7;
  bf16x8 fa[2][C::VB], fb[2][C::MB];
  // the wave's 32-row blocks of hidden rows that hold live rows (all MB but in the
  // last row tile); a block with none is neither read nor multiplied
  const int mlive = __builtin_amdgcn_readfirstlane(
      min(C::MB, max(0, (mrows - wm * C::MW + 31) / 32)));
  auto rd = [&]<int ST, int KS, int BUF, bool GUARD>() {
    if (GUARD && mlive == 0) return;
    const unsigned char* As = smem + ST * C::STAGE + (wv * C::VW) * kRowBytes + frag_base;
    const unsigned char* Bs = smem + ST * C::STAGE + (VT + wm * C::MW) * kRowBytes + frag_base;
    const int slot = (((2 * KS + h2) ^ fsw) << 4);
#pragma unroll
    for (int vb = 0; vb < C::VB; ++vb)
      fa[BUF][vb] = *reinterpret_cast<const bf16x8*>(As + vb * 32 * kRowBytes + slot);
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
      if (!GUARD || mb < mlive)
        fb[BUF][mb] = *reinterpret_cast<const bf16x8*>(Bs + mb * 32 * kRowBytes + slot);
  };
  auto mfmas = [&]<int BUF, bool GUARD>() {
#pragma unroll
    for (int vb = 0; vb < C::VB; ++vb)
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb)
        if (!GUARD || mb < mlive)
          acc[vb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[BUF][vb], fb[BUF][mb], acc[vb][mb], 0, 0, 0);
  };
  // the reads of the next substep between this substep's MFMAs, one after each MFMA
  auto interleave = [&]() {
#pragma unroll
    for (int i = 0; i < C::VB + C::MB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, C::VB * C::MB - (C::VB + C::MB), 0);
  };
  // vmcnt(n) with the other counters left at their maxima
  constexpr int kWaitOne = 0x0f70 | (C::PER_WAVE & 15) | ((C::PER_WAVE >> 4) << 14);

  // Step s of stage ST (= s mod NS): substeps 0..2 each run their MFMAs with the next
  // substep's fragments read in between.  Then, with substep 3's fragments in
  // registers, the wave waits for its loads of step s + 1 and meets the barrier: every
  // wave then holds what it needs of stage ST, which is refilled with step s + NS, and
  // step s + 1's rows are visible, so its first fragments are read while substep 3's
  // MFMAs run.
  auto step = [&]<int ST, bool GUARD>(int s) {
    rd.template operator()<ST, 1, 1, GUARD>();
    mfmas.template operator()<0, GUARD>();
    interleave();
    rd.template operator()<ST, 2, 0, GUARD>();
    mfmas.template operator()<1, GUARD>();
    interleave();
    rd.template operator()<ST, 3, 1, GUARD>();
    mfmas.template operator()<0, GUARD>();
    interleave();
    if (s + 1 < nk) {
      if (NS == 3 && s + 2 < nk)
        __builtin_amdgcn_s_waitcnt(kWaitOne & ~0x0f00);   // lgkmcnt(0), vmcnt(PER_WAVE)
      else
        __builtin_amdgcn_s_waitcnt(0x0070);               // lgkmcnt(0), vmcnt(0)
      __builtin_amdgcn_s_barrier();
      if (s + NS < nk) issue.template operator()<ST>(s + NS);
      rd.template operator()<(ST + 1) % NS, 0, 0, GUARD>();
    }
    mfmas.template operator()<1, GUARD>();
  };

  // prologue: the first NS steps in flight, then step 0's rows
  issue.template operator()<0>(0);
  if (1 < nk) issue.template operator()<1 % NS>(1);
  if (NS == 3 && 2 < nk) issue.template operator()<2 % NS>(2);
  const int later = min(NS - 1, nk - 1);
  if (later == 0) __builtin_amdgcn_s_waitcnt(0x0f70);
  else if (later == 1) __builtin_amdgcn_s_waitcnt(kWaitOne);
  else __builtin_amdgcn_s_waitcnt(0x0f70 | ((2 * C::PER_WAVE) & 15) | (((2 * C::PER_WAVE) >> 4) << 14));
  __builtin_amdgcn_s_barrier();
  auto kloop = [&]<bool GUARD>() {
    rd.template operator()<0, 0, 0, GUARD>();
    for (int s = 0; s < nk; s += NS) {
      step.template operator()<0, GUARD>(s);
      if (s + 1 < nk) step.template operator()<1 % NS, GUARD>(s + 1);
      if (NS == 3 && s + 2 < nk) step.template operator()<2 % NS, GUARD>(s + 2);
    }
  };
  if (mlive == C::MB)
    kloop.template operator()<false>();
  else
    kloop.template operator()<true>();

  // ---- epilogue.  Lane l holds, for column block mb, hidden row wm*MW + mb*32 + l%32
  // against vocabulary rows wv*VW + vb*32 + 8(r/4) + 4 h2 + r%4: visited in increasing
  // order, so a strict comparison keeps the smaller id among equal values.
  __syncthreads();  // every wave is done with the ring: its LDS holds the wave partials
  Partial* red = reinterpret_cast<Partial*>(smem);  // [NWV][MT]
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) {
    float bv = -INFINITY;
    int bi = INT32_MAX;
#pragma unroll
    for (int vb = 0; vb < C::VB; ++vb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int v = wv * C::VW + vb * 32 + 8 * (r / 4) + 4 * h2 + (r % 4);
        const float x = acc[vb][mb][r];
        if (v < vrows && x > bv) {
          bv = x;
          bi = v0 + v;
        }
      }
    const float ov = xchg<32>(bv);
    const int oi = xchg<32>(bi);
    if (better(ov, oi, bv, bi)) {
      bv = ov;
      bi = oi;
    }
    if (h2 == 0) red[wv * MT + wm * C::MW + mb * 32 + l32] = Partial{bv, bi};
  }
  __syncthreads();
  for (int m = tid; m < mrows; m += C::NW * 64) {
    Partial p = red[m];
#pragma unroll
    for (int w = 1; w < NWV; ++w) {
      const Partial o = red[w * MT + m];
      if (better(o.v, o.i, p.v, p.i)) p = o;
    }
    partial[(int64_t)(m0 + m) * nvt + vt] = p;
  }
}

// One wave per hidden row: the best of its vocabulary tiles' partials; padding nodes
// (n >= num_nodes[s]) get -1 and -inf.
__global__ void __launch_bounds__(256)
lm_head_reduce(const Partial* __restrict__ partial, int M, int N, int nvt,
               const int32_t* __restrict__ num_nodes, int32_t* __restrict__ node_tok,
               float* __restrict__ node_max) {
  const int m = blockIdx.x * 4 + threadIdx.x / 64;
  if (m >= M) return;
  const int lane = threadIdx.x % 64;
  const int s = m / N, n = m % N;
  if (num_nodes && n >= num_nodes[s]) {
    if (lane == 0) {
      node_tok[m] = -1;
      if (node_max) node_max[m] = -INFINITY;
    }
    return;
  }
  float bv = -INFINITY;
  int bi = INT32_MAX;
  for (int j = lane; j < nvt; j += 64) {
    const Partial p = partial[(int64_t)m * nvt + j];
    if (better(p.v, p.i, bv, bi)) {
      bv = p.v;
      bi = p.i;
    }
  }
  wave_argmax(bv, bi);
  if (lane == 0) {
    node_tok[m] = bi;
    if (node_max) node_max[m] = bv;
  }
}

// One wave per sequence: from the root, move to the child (smallest index first) whose
// token is the current node's target token, until there is none.
__global__ void __launch_bounds__(64)
tree_walk_tokens_kernel(const int32_t* __restrict__ tree_tok, const int32_t* __restrict__ parent,
                        const int32_t* __restrict__ num_nodes, const int32_t* __restrict__ node_tok,
                        int N, int L, int32_t* __restrict__ accept_len, int32_t* __restrict__ acc_nodes,
                        int32_t* __restrict__ acc_tok, int32_t* __restrict__ bonus_out) {
  const int s = blockIdx.x;
  const int lane = threadIdx.x;
  const int nn = min(max(num_nodes[s], 1), N);
  const int32_t* tt = tree_tok + (int64_t)s * N;
  const int32_t* pp = parent + (int64_t)s * N;
  int cur = 0, a = 0;
  int want = node_tok[(int64_t)s * N];
  while (a < L) {
    // the smallest-index child of cur carrying want: 64 candidates per ballot
    int nxt = -1;
    for (int base = 0; base < nn && nxt < 0; base += 64) {
      const int c = base + lane;
      const unsigned long long hit = ballot(c < nn && pp[c] == cur && tt[c] == want);
      if (hit) nxt = base + __builtin_ctzll(hit);
    }
    if (nxt < 0) break;
    if (lane == 0) {
      acc_nodes[(int64_t)s * L + a] = nxt;
      acc_tok[(int64_t)s * L + a] = tt[nxt];
    }
    ++a;
    cur = nxt;
    want = node_tok[(int64_t)s * N + cur];
  }
  for (int j = a + lane; j < L; j += 64) {
    acc_nodes[(int64_t)s * L + j] = -1;
    acc_tok[(int64_t)s * L + j] = -1;
  }
  if (lane == 0) {
    accept_len[s] = a;
    bonus_out[s] = want;
  }
}

template <int VT, int MT, int NWV, int NWM, int NS>
hipError_t launch_tiles(const void* H, const void* W, int M, int V, int d, Partial* part,
                        hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  using C = LmCfg<VT, MT, NWV, NWM, NS>;
  const int nvt = (int)ceil_div(V, VT), nmt = (int)ceil_div(M, MT);
  const int per_xcd = (int)ceil_div((int64_t)nvt * nmt, 8);
  hipExtLaunchKernelGGL((lm_head_tiles<VT, MT, NWV, NWM, NS>), dim3(8 * per_xcd), dim3(C::NW * 64), 0,
                        st, ev0, ev1, 0, (const bf16_t*)H, (const bf16_t*)W, M, V, d, nvt, nmt,
                        per_xcd, part);
  return hipGetLastError();
}

}  // namespace

LmPlan lm_head_plan(int S, int B, int64_t vocab, int d) {
  LmPlan p{};
  const int64_t M = (int64_t)S * (B + 1);
  p.vt = 256;
  p.mt = M > 128 ? 256 : M > 64 ? 128 : M > 32 ? 64 : 32;
  p.nvt = (int)ceil_div(vocab, p.vt);
  p.ws_bytes = align_up((size_t)M * p.nvt * sizeof(Partial), 256);
  (void)d;
  return p;
}

hipError_t launch_lm_head(const void* hidden, const void* weight, const int32_t* num_nodes, int S,
                          int B, int d, int64_t vocab, int32_t* node_tok, float* node_max,
                          void* ws, const LmPlan& p, hipStream_t st) {
  const int N = B + 1;
  const int M = S * N;
  const int V = (int)vocab;
  Partial* part = (Partial*)ws;
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  if (!lm_prof_events(&ev0, &ev1)) ev0 = ev1 = nullptr;
  hipError_t e;
  switch (p.mt) {
    case 256: e = launch_tiles<256, 256, 2, 4, 2>(hidden, weight, M, V, d, part, st, ev0, ev1); break;
    case 128: e = launch_tiles<256, 128, 2, 2, 3>(hidden, weight, M, V, d, part, st, ev0, ev1); break;
    case 64: e = launch_tiles<256, 64, 4, 1, 2>(hidden, weight, M, V, d, part, st, ev0, ev1); break;
    default: e = launch_tiles<256, 32, 4, 1, 2>(hidden, weight, M, V, d, part, st, ev0, ev1); break;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lm_head_reduce, dim3((unsigned)ceil_div(M, 4)), dim3(256), 0, st, part, M, N,
                     p.nvt, num_nodes, node_tok, node_max);
  return hipGetLastError();
}

hipError_t launch_tree_walk_tokens(const int32_t* tree_tok, const int32_t* parent,
                                   const int32_t* num_nodes, const int32_t* node_tok, int S, int B,
                                   int L, int32_t* accept_len, int32_t* acc_nodes, int32_t* acc_tok,
                                   int32_t* bonus_out, hipStream_t st) {
  hipLaunchKernelGGL(tree_walk_tokens_kernel, dim3(S), dim3(64), 0, st, tree_tok, parent, num_nodes,
                     node_tok, B + 1, L, accept_len, acc_nodes, acc_tok, bonus_out);
  return hipGetLastError();
}

}  // namespace ddt
