// Expert-indexed MoE decode pair (moe_gemv page, module docstring and the
// gate_up / down_combine docstrings), expert-major: every routed expert's
// weights are read once per call, for all the tokens routed to it.
//
// Routing.  Every workgroup rebuilds the call's routing in LDS from ids (at
// most 32 tokens x 16 slots = 512 pairs): the distinct experts in order of
// first appearance ("slots"), and the pairs of every slot in ascending pair
// order.  No host synchronization and no workspace are needed, and the order
// of every floating-point sum depends on ids alone.
//
//   gate_up routed: act[p][i] = bf16(silu(g) * u),  g, u = FP32 sum * alpha[e]
//   gate_up shared: sact[t][i] = bf16(silu(bf16(g)) * bf16(u)),  g, u = FP32 sum * gssh
//   down_combine:   y = bf16(FP32 sum * alpha2[e]) per pair,
//                   out = bf16(bf16(sum of tw * y) + y_shared)
//
// Two forms of each kernel:
//
// VALU forms (M <= 2).  Chunk-interleaved loads and per-token dot products
// (chunk_core.hpp).  gate_up walks persistent items (slot, quad of gate rows
// and the matching up rows) with four waves splitting H and meeting in LDS;
// down_combine gives a workgroup a quad of H rows, its waves take the slots
// round robin and stream their jobs (slot, token group, K block) through a
// two-slot ring of registers.
//
// MFMA forms (M >= 3).  The swap-AB MFMA building blocks of the dense GEMV
// (mfma_core.hpp) with each slot's tokens gathered by the loads that stage
// activations in LDS; the dequant then costs the same for any number of
// tokens.  Each wave streams whole work units through one LDS ring (see the
// section below).
//
// Inside every ring the loads are counted: no other vector memory access may
// fall between them, and LDS tables are read with lds_read_u32 so that the
// compiler adds no wait for the loads still writing ring slots.
#include "chunk_core.hpp"
#include "device_common.hpp"
#include "launch.hpp"
#include "mfma_core.hpp"
#include "unit_core.hpp"

namespace w4a16 {

constexpr int kMoeMaxPairs = 512;  // 32 tokens x 16 slots
constexpr int kMoeMaxTokens = 32;

__device__ __forceinline__ int clamp_expert(int32_t id, int E) {
  return id < 0 ? 0 : (id >= E ? E - 1 : id);
}

// Values the whole wave agrees on, moved to scalar registers (the compiler
// cannot always prove that values read from LDS are uniform, and a buffer
// resource built from a value it deems divergent becomes a per-lane loop).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const void*>((static_cast<uint64_t>(hi) << 32) | lo);
}
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
  return static_cast<const uint8_t*>(uniform_ptr(static_cast<const void*>(p)));
}
__device__ __forceinline__ int64_t uniform_i64(int64_t v) {
  return static_cast<int64_t>(reinterpret_cast<uint64_t>(uniform_ptr(reinterpret_cast<const void*>(v))));
}
// c ? a : b on values: a conditional between two named variables is an
// lvalue, which the compiler may turn into a load from a chosen address and
// so keep those variables in scratch memory.
template <typename T>
__device__ __forceinline__ T pick(bool c, T a, T b) {
  return c ? a : b;
}
__device__ __forceinline__ rsrc_t uniform_rsrc(const void* base, uint32_t bytes) {
  return make_rsrc(uniform_ptr(base), __builtin_amdgcn_readfirstlane(bytes));
}

constexpr int kMoeExpertTable = 2048;  // experts with an LDS first-pair entry

struct alignas(16) MoeRouting {
  int32_t id[kMoeMaxPairs];         // clamped expert of every pair (-1 past P)
  int32_t first[kMoeMaxPairs];      // pair -> first pair routed to the same expert
  int32_t within[kMoeMaxPairs];     // pair -> rank among that expert's pairs
  int32_t fslot[kMoeMaxPairs];      // first pair -> its slot
  int32_t expert[kMoeMaxPairs];     // slot -> expert
  int32_t count[kMoeMaxPairs];      // slot -> number of pairs
  int32_t start[kMoeMaxPairs + 1];  // slot -> offset into order
  int32_t order[kMoeMaxPairs];      // pairs grouped by slot, ascending within a slot
  float tw[kMoeMaxPairs];           // pair -> routing weight (down_combine)
  int32_t first_of[kMoeExpertTable];  // expert -> first pair (E <= kMoeExpertTable)
  int32_t chunk_firsts[kMoeMaxPairs / 64];
  int32_t D;                        // distinct experts
};

// The routing the VALU forms need for their at most 2 x 16 pairs (the fields
// of MoeRouting they read), about 0.7 KB of LDS instead of 26 KB, so that
// LDS does not bound how many of their workgroups a compute unit holds.
constexpr int kMoeValuMaxPairs = 32;
struct alignas(16) MoeRoutingSmall {
  int32_t expert[kMoeValuMaxPairs];
  int32_t count[kMoeValuMaxPairs];
  int32_t start[kMoeValuMaxPairs + 1];
  int32_t order[kMoeValuMaxPairs];
  float tw[kMoeValuMaxPairs];
  int32_t D;
};

// Number of i in [lo, hi) with a[i] == v: a scan of an LDS array in blocks of
// 16 entries read as four 16-byte broadcasts (the array is readable up to
// kMoeMaxPairs; entries outside [lo, hi) are masked).
__device__ __forceinline__ int count_equal(const int32_t* a, int lo, int hi, int v) {
  int n = 0;
  for (int b = lo & ~15; b < hi; b += 16) {
    const int4* q = reinterpret_cast<const int4*>(a + b);
    const int4 x0 = q[0], x1 = q[1], x2 = q[2], x3 = q[3];
    const int e[16] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w,
                       x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
#pragma unroll
    for (int k = 0; k < 16; ++k) n += (b + k >= lo && b + k < hi && e[k] == v) ? 1 : 0;
  }
  return n;
}

// Sum of a[0..hi) (same blocked reads).
__device__ __forceinline__ int sum_prefix(const int32_t* a, int hi) {
  int n = 0;
  for (int b = 0; b < hi; b += 16) {
    const int4* q = reinterpret_cast<const int4*>(a + b);
    const int4 x0 = q[0], x1 = q[1], x2 = q[2], x3 = q[3];
    const int e[16] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w,
                       x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
#pragma unroll
    for (int k = 0; k < 16; ++k) n += (b + k < hi) ? e[k] : 0;
  }
  return n;
}

// Builds the routing of P pairs with the whole workgroup; tw (may be null)
// is loaded together with ids.  Ends with a barrier.
//   first pair of every expert: an atomicMin per pair into an LDS table (E up
//     to kMoeExpertTable; larger E falls back to a scan of the earlier pairs);
//   slot of a first pair: number of first pairs before it, from 64-pair
//     ballots; within-expert rank: number of earlier pairs with that expert.
__device__ void build_routing(MoeRouting& r, const int32_t* ids, const float* tw, int P, int E) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int lane = tid & 63, wave = tid >> 6, nwaves = nt >> 6;
  const bool table = E <= kMoeExpertTable;
  if (table)
    for (int e = tid; e < E; e += nt) r.first_of[e] = kMoeMaxPairs;
  for (int p = tid; p < kMoeMaxPairs; p += nt) {
    r.id[p] = p < P ? clamp_expert(ids[p], E) : -1;
    if (tw && p < P) r.tw[p] = tw[p];
    r.count[p] = 0;
  }
  __syncthreads();
  if (table)
    for (int p = tid; p < P; p += nt) atomicMin(&r.first_of[r.id[p]], p);
  __syncthreads();
  for (int p = tid; p < P; p += nt) {
    const int e = r.id[p];
    const int within = count_equal(r.id, 0, p, e);
    int first = p;
    if (table) {
      first = r.first_of[e];
    } else if (within > 0) {
      for (int q = 0; q < p; ++q) {
        if (r.id[q] == e) {
          first = q;
          break;
        }
      }
    }
    r.first[p] = first;
    r.within[p] = within;
  }
  __syncthreads();
  // slots: ranks of the first pairs, chunk by chunk of 64 pairs
  const int nchunks = (P + 63) / 64;
  for (int c = wave; c < nchunks; c += nwaves) {
    const int p = c * 64 + lane;
    const bool f = p < P && r.first[p] == p;
    const uint64_t mask = __ballot(f);
    if (lane == 0) r.chunk_firsts[c] = __popcll(mask);
  }
  __syncthreads();
  for (int c = wave; c < nchunks; c += nwaves) {
    const int p = c * 64 + lane;
    const bool f = p < P && r.first[p] == p;
    const uint64_t mask = __ballot(f);
    int before = __popcll(mask & ((uint64_t(1) << lane) - 1));
    for (int c2 = 0; c2 < c; ++c2) before += r.chunk_firsts[c2];
    if (f) {
      r.fslot[p] = before;
      r.expert[before] = r.id[p];
    }
  }
  if (tid == 0) {
    int d = 0;
    for (int c = 0; c < nchunks; ++c) d += r.chunk_firsts[c];
    r.D = d;
  }
  __syncthreads();
  for (int p = tid; p < P; p += nt) atomicAdd(&r.count[r.fslot[r.first[p]]], 1);
  __syncthreads();
  const int D = r.D;
  for (int s = tid; s <= D; s += nt) r.start[s] = sum_prefix(r.count, s);
  __syncthreads();
  for (int p = tid; p < P; p += nt) r.order[r.start[r.fslot[r.first[p]]] + r.within[p]] = p;
  __syncthreads();
}

// The same routing for at most 64 pairs (one per lane of the first wave),
// with cross-lane reads instead of LDS tables: the other waves only wait at
// the closing barrier.  The VALU forms (one or two tokens: at most 32 pairs)
// use it; a decode step's few pairs then cost a handful of scalar loops
// instead of the table passes and their barriers (measured 0.5 / 0.8 us off
// gate_up / down_combine at one token).  The MFMA forms keep the table
// builder: with both builders in them they ran 12-16% slower at 8 and 32
// tokens.
template <typename Routing>
__device__ void build_routing_wave(Routing& r, const int32_t* ids, const float* tw, int P, int E) {
  if (threadIdx.x < 64) {
    const int p = threadIdx.x;
    const bool live = p < P;
    // absent pairs get distinct negative ids, so they match nothing
    const int e = live ? clamp_expert(ids[p], E) : -1 - p;
    int first = p, within = 0;
    for (int q = 0; q < P; ++q) {
      const int eq = __builtin_amdgcn_readlane(e, q);
      if (q < p && eq == e) {
        ++within;
        first = q < first ? q : first;
      }
    }
    const bool is_first = live && first == p;
    const uint64_t firsts = __ballot(is_first);
    const int slot_if_first = __popcll(firsts & ((uint64_t(1) << p) - 1));
    int count = 0;
    for (int q = 0; q < P; ++q) count += __builtin_amdgcn_readlane(first, q) == p ? 1 : 0;
    // start of a first pair's slot: the counts of the first pairs before it
    int start = 0;
    for (int q = 0; q < P; ++q) {  // a uniform loop: q is the same on every lane
      const int fq = __builtin_amdgcn_readlane(first, q);
      const int cq = __builtin_amdgcn_readlane(count, q);
      start += (q < p && fq == q) ? cq : 0;
    }
    const int my_start = __shfl(start, first);
    if (is_first) {
      r.expert[slot_if_first] = e;
      r.count[slot_if_first] = count;
      r.start[slot_if_first] = start;
    }
    if (live) {
      r.order[my_start + within] = p;
      if (tw) r.tw[p] = tw[p];
    }
    if (p == 0) {
      r.D = __popcll(firsts);
      r.start[__popcll(firsts)] = P;
    }
  }
  __syncthreads();
}


// ------------------------------------------------------------------ gate_up
// Work items are (slot, gate quad of the expert's I rows) and (gate quad of
// the shared expert's SI rows); a persistent grid builds the routing once per
// workgroup and walks the items.  For an item, the four waves split H; the
// expert's gate and up quads are read once (per K block) and applied to the
// slot's tokens MT at a time.  Each item is straight-line: all of its loads
// are issued before its arithmetic, and its results are stored before the
// next item's loads (so no wait ever mixes stores and loads in flight).
template <int MT, int C>
__global__ __launch_bounds__(256) void k_moe_gate_up(const MoeGateUpParams p) {
  constexpr int KS = 4;                 // waves per item, each a slice of H
  constexpr int PV = 2;                 // gate, up
  constexpr int V = MT * 4 * PV;        // value index (m * 4 + q) * 2 + u
  using RS = ReduceScatter<V, PV>;
  __shared__ MoeRoutingSmall rt;
  __shared__ float red[KS - 1][RS::LEFT][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int kw = uniform(tid >> 6);
  const int P = p.M * p.topk;  // at most 2 x 16: one wave builds the routing
  build_routing_wave(rt, p.ids, nullptr, P, p.E);
  const int D = uniform(rt.D);
  // 32-bit item bookkeeping: at most 512 slots x (I / 4) quads
  const int units_r = (p.I + 127) / 128 * 32;
  const int units_s = (p.SI + 127) / 128 * 32;
  const int items = D * units_r + units_s;
  const uint32_t nch = p.H / 8;
  const int nkb = static_cast<int>((nch + KS * C * 64 - 1) / (KS * C * 64));
  const uint32_t shift = 8u * ((lane >> 1) & 3);
  const uint32_t row_bytes = p.H / 2;
  const uint32_t tiles = p.H / 64;
  const rsrc_t rx = make_rsrc(p.x, static_cast<uint32_t>(p.M) * p.H * 2);
  const float gssh = *p.gssh;

  for (int item = xcd_logical_block(); item < items; item += gridDim.x) {
    const bool shared = item >= D * units_r;
    const int s = shared ? 0 : item / units_r;
    const int u = shared ? item - D * units_r : item - s * units_r;
    const int e = shared ? 0 : uniform(rt.expert[s]);
    const int cnt = shared ? p.M : uniform(rt.count[s]);
    const int first = shared ? 0 : uniform(rt.start[s]);
    const int half = shared ? p.SI : p.I;
    const float scale = shared ? gssh : p.alpha[e];
    int64_t rows[8];
    bool rv[8];
    quad_rows<8>(u, half, half, rows, rv);
    const bool quad_ok[2] = {true, half % 128 == 0};
    const rsrc_t rw = uniform_rsrc(shared ? p.wsh : p.w1 + e * p.w1_expert_bytes,
                                   static_cast<uint32_t>(shared ? p.wsh_bytes : p.w1_expert_bytes));
    const rsrc_t rs = uniform_rsrc(shared ? p.ssh : p.w1s + e * p.s1_expert_bytes,
                                   static_cast<uint32_t>(shared ? p.ssh_bytes : p.s1_expert_bytes));

    for (int g0 = 0; g0 < cnt; g0 += MT) {
      // token rows of this group (pairs of the slot in ascending order)
      uint32_t xoff[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const int idx = g0 + m;
        const int t = shared ? idx : rt.order[first + (idx < cnt ? idx : cnt - 1)] / p.topk;
        xoff[m] = off_if(idx < cnt, static_cast<uint32_t>(t) * p.H * 2);
      }
      float acc[8][MT];
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[i][m] = 0.0f;
      for (int kb = 0; kb < nkb; ++kb) {
        uint32_t ch[C];
        bool ok[C];
#pragma unroll
        for (int q = 0; q < C; ++q) {
          ch[q] = static_cast<uint32_t>((kb * KS + kw) * C + q) * 64 + lane;
          ok[q] = ch[q] < nch;
        }
        ChunkX<C, MT> xb;
        ChunkW<C, 8> wb;
        chunk_issue_x<C, MT>(xb, rx, xoff, ch, ok);
        chunk_issue_w<C, 8>(wb, rw, row_bytes, rs, tiles, rows, rv, quad_ok, ch, ok);
        __builtin_amdgcn_sched_barrier(0);  // every load ahead of the arithmetic
        chunk_compute<C, 8, MT>(wb, xb, shift, acc);
      }
      float v[V];
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int w = 0; w < PV; ++w) v[(m * 4 + q) * PV + w] = acc[4 * w + q][m];
      reduce_scatter<V, PV>(v);
      if (kw > 0) {
#pragma unroll
        for (int i = 0; i < RS::LEFT; ++i) red[kw - 1][i][lane] = v[i];
      }
      __syncthreads();
      if (kw == 0) {
#pragma unroll
        for (int w = 0; w < KS - 1; ++w)
#pragma unroll
          for (int i = 0; i < RS::LEFT; ++i) v[i] += red[w][i][lane];
        const int base = reduce_scatter_base<V, PV>(lane);
#pragma unroll
        for (int i = 0; i < RS::LEFT / PV; ++i) {
          const int vi = base + i * PV;
          const int m = vi / (4 * PV), q = (vi / PV) % 4;
          const int idx = g0 + m;
          const int64_t row = static_cast<int64_t>(u >> 5) * 128 + (u & 31) + 32 * q;
          if ((lane & 15) == i && idx < cnt && row < half) {
            float g = v[i * PV] * scale, up = v[i * PV + 1] * scale;
            if (shared) {
              g = bf16_bits_to_f32(f32_to_bf16_bits(g));
              up = bf16_bits_to_f32(f32_to_bf16_bits(up));
              p.sact[static_cast<int64_t>(idx) * p.SI + row] = f32_to_bf16_bits(silu_f32(g) * up);
            } else {
              const int pair = rt.order[first + idx];
              p.act[static_cast<int64_t>(pair) * p.I + row] = f32_to_bf16_bits(silu_f32(g) * up);
            }
          }
        }
      }
      __syncthreads();
    }
  }
}

// ------------------------------------------------------------------ down_combine
template <int MT, int C, int NW>
__global__ __launch_bounds__(NW * 64) void k_moe_down_combine(const MoeDownParams p) {
  constexpr int V = MT * 4;  // value index m * 4 + q
  using RS = ReduceScatter<V, 1>;
  __shared__ MoeRoutingSmall rt;
  __shared__ float part[NW][kMoeMaxTokens][4];
  __shared__ float ysh[kMoeMaxTokens][4];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int P = p.M * p.topk;  // at most 2 x 16: one wave builds the routing
  build_routing_wave(rt, p.ids, p.tw, P, p.E);
  const int D = uniform(rt.D);
  const float gssd = *p.gssd;
  const int64_t units = (p.H + 127) / 128 * 32;
  const uint32_t shift = 8u * ((lane >> 1) & 3);
  const uint32_t act_bytes = static_cast<uint32_t>(P) * p.I * 2;
  const uint32_t sact_bytes = static_cast<uint32_t>(p.M) * p.SI * 2;

  // Job = (slot s, group of MT tokens from g0, K block kb); wave w takes the
  // slots s = w, w + NW, ...; slot D is the shared expert.
  struct Job {
    int s, g0, kb;
  };
  auto npairs_of = [&](int s) -> int {
    const int cnt = uniform(rt.count[s < D ? s : D - 1]);
    return s < D ? cnt : p.M;
  };
  auto nkb_of = [&](int s) -> int {
    const int k = s < D ? p.I : p.SI;
    return (k / 8 + C * 64 - 1) / (C * 64);
  };
  auto advance = [&](Job j) -> Job {
    if (++j.kb == nkb_of(j.s)) {
      j.kb = 0;
      j.g0 += MT;
      if (j.g0 >= npairs_of(j.s)) {
        j.g0 = 0;
        j.s += NW;
      }
    }
    return j;
  };
  int njobs = 0;
  for (int s = wave; s <= D; s += NW) njobs += (npairs_of(s) + MT - 1) / MT * nkb_of(s);

  for (int64_t u = xcd_logical_block(); u < units; u += gridDim.x) {
    int64_t rows[4];
    bool rv[4];
    quad_rows<4>(u, p.H, 0, rows, rv);
    for (int i = lane; i < p.M * 4; i += 64) part[wave][i >> 2][i & 3] = 0.0f;

    auto issue = [&](const Job& j, ChunkW<C, 4>& wb, ChunkX<C, MT>& xb) {
      const bool valid = j.s <= D;
      const bool shared = j.s == D;
      const int e = uniform(rt.expert[j.s < D ? j.s : D - 1]);
      const int k = shared ? p.SI : p.I;
      const uint32_t nch = k / 8;
      uint32_t ch[C];
      bool ok[C];
#pragma unroll
      for (int q = 0; q < C; ++q) {
        ch[q] = static_cast<uint32_t>(j.kb * C + q) * 64 + lane;
        ok[q] = valid && ch[q] < nch;
      }
      const int np = valid ? npairs_of(j.s) : 0;
      const int first = rt.start[j.s < D ? j.s : D];
      uint32_t xoff[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const int idx = j.g0 + m;
        const int o = first + idx;
        const int row = shared ? idx : rt.order[o < P ? o : P - 1];
        xoff[m] = off_if(idx < np, static_cast<uint32_t>(row) * k * 2);
      }
      chunk_issue_x<C, MT>(xb, uniform_rsrc(shared ? static_cast<const void*>(p.sact) : static_cast<const void*>(p.act),
                                            shared ? sact_bytes : act_bytes),
                           xoff, ch, ok);
      const bool quad_ok[1] = {true};
      const uint8_t* wbase = shared ? p.wsd : p.w2 + e * p.w2_expert_bytes;
      const uint8_t* sbase = shared ? p.ssd : p.w2s + e * p.s2_expert_bytes;
      const uint32_t wbytes = static_cast<uint32_t>(shared ? p.wsd_bytes : p.w2_expert_bytes);
      const uint32_t sbytes = static_cast<uint32_t>(shared ? p.ssd_bytes : p.s2_expert_bytes);
      chunk_issue_w<C, 4>(wb, uniform_rsrc(wbase, wbytes), k / 2, uniform_rsrc(sbase, sbytes), k / 64, rows, rv,
                          quad_ok, ch, ok);
      __builtin_amdgcn_sched_barrier(0);  // as in k_moe_gate_up
    };

    float acc[4][MT];
    auto finish = [&](const Job& j) {
      const bool shared = j.s == D;
      // a scalar load: it does not count against the vector loads in flight
      const float scale = shared ? gssd : p.alpha2[uniform(rt.expert[j.s < D ? j.s : D - 1])];
      const int np = npairs_of(j.s);
      const int first = rt.start[j.s < D ? j.s : D];
      float v[V];
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int q = 0; q < 4; ++q) v[m * 4 + q] = acc[q][m];
      reduce_scatter<V, 1>(v);
      const int base = reduce_scatter_base<V, 1>(lane);
      // one token at a time: two pairs of one token routed to the same
      // expert must not update its partial in the same instruction
#pragma unroll
      for (int mm = 0; mm < MT; ++mm) {
#pragma unroll
        for (int i = 0; i < RS::LEFT; ++i) {
          const int vi = base + i;
          const int m = vi / 4, q = vi % 4;
          const int idx = j.g0 + m;
          if (m == mm && (lane & 15) == i && idx < np) {
            const float y = bf16_bits_to_f32(f32_to_bf16_bits(v[i] * scale));
            if (shared) {
              ysh[idx][q] = y;
            } else {
              const int pair = rt.order[first + idx];
              part[wave][pair / p.topk][q] += rt.tw[pair] * y;
            }
          }
        }
      }
    };

    ChunkW<C, 4> wa, wb;
    ChunkX<C, MT> xa, xb;
    Job ja{wave, 0, 0};
    Job jb = advance(ja);
    issue(ja, wa, xa);
    issue(jb, wb, xb);  // jobs past the last slot read nothing
    auto consume = [&](const Job& j, const ChunkW<C, 4>& w, const ChunkX<C, MT>& x) {
      if (j.kb == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int m = 0; m < MT; ++m) acc[i][m] = 0.0f;
      }
      chunk_compute<C, 4, MT>(w, x, shift, acc);
      if (j.kb == nkb_of(j.s) - 1) finish(j);
    };
    for (int i = 0; i < njobs; i += 2) {
      consume(ja, wa, xa);
      ja = advance(jb);
      issue(ja, wa, xa);
      if (i + 1 < njobs) consume(jb, wb, xb);
      jb = advance(ja);
      issue(jb, wb, xb);
    }
    __syncthreads();
    for (int i = tid; i < p.M * 4; i += blockDim.x) {
      const int t = i >> 2, q = i & 3;
      const int64_t row = (u >> 5) * 128 + (u & 31) + 32 * q;
      if (row < p.H) {
        float s = part[0][t][q];
#pragma unroll
        for (int w = 1; w < NW; ++w) s += part[w][t][q];  // in wave order
        const float sr = bf16_bits_to_f32(f32_to_bf16_bits(s));
        p.out[static_cast<int64_t>(t) * p.H + row] = f32_to_bf16_bits(sr + ysh[t][q]);
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ MFMA forms
// For M >= 2 both kernels use the swap-AB MFMA building blocks of the dense
// GEMV (mfma_core.hpp): 16 weight rows are the A operand, up to XT tokens of
// one slot the B operand, staged through a per-wave LDS ring by loads that
// gather the slot's rows.  The dequant costs the same for any number of
// tokens, where the VALU forms pay one dot product per token.
//
// Each wave owns a stream of jobs (work unit, group of XT tokens, 128-k
// step) and runs the whole K of a unit itself, so nothing is reduced across
// waves.  One ring of kMoeRing steps runs through all of a wave's jobs: a
// slot is consumed, its LDS reads retired, and it is refilled with the job
// kMoeRing ahead, so every wait counts the same loads; the last round drains
// the ring without refilling it.  A job's results are written by the wave
// that consumed its last step.  Two steps in flight per wave measured as fast
// as four or eight, and leave LDS for more resident waves.
constexpr int kMoeRing = 2;
constexpr int kMoeDownRing = 2;
constexpr int kMoeDownWaves = 12;
constexpr int kMoeGateUpWaves = 4;

// The job the wave issues next, and what a ring slot remembers of the job it
// holds.  All fields are wave-uniform.
struct MoeJob {
  int unit;      // work unit (kernel-specific), < 0 once the stream is over
  int slot;      // routing slot (== D: the shared expert)
  int tile;      // 16-row tile
  int cnt;       // tokens (pairs) of the slot
  int first;     // offset of the slot's pairs in the routing order
  int g0;        // first token of the group
  int step;      // 128-k step within the unit
  int nsteps;    // steps of the unit
  float scale;   // alpha of the expert (or the shared global scale)
  int expert;    // expert of the slot (0 for the shared expert)
};

// Job arithmetic shared by both kernels: next step, next group, next unit.
template <int XT>
__device__ __forceinline__ bool moe_job_next(MoeJob& j) {
  if (++j.step < j.nsteps) return false;
  j.step = 0;
  j.g0 += XT;
  return j.g0 >= j.cnt;  // the unit is done: the caller moves to its next one
}

// gate_up.  Work unit u = (slot, 16-row tile of its gate rows): the A
// operands are the gate tile and the matching up tile (rows + half); units
// u, u + (all waves), ... belong to one wave.
//   routed: act[p][i] = bf16(silu(g) * u),  g, u = FP32 sum * alpha[e]
//   shared: sact[t][i] = bf16(silu(bf16(g)) * bf16(u)),  g, u = FP32 sum * gssh
template <int XT>
__global__ __launch_bounds__(kMoeGateUpWaves * 64) void k_moe_gate_up_mfma(const MoeGateUpParams p) {
  constexpr int W = kMoeGateUpWaves, D = kMoeRing, NA = 2, CPT = 16, LX = XT * CPT / 64, PER = 2;
  constexpr int L = LX + NA * PER;              // loads per step
  constexpr int FULL_AFTER = NA * PER + (D - 1) * L;
  constexpr int SLOT = XT * CPT;                // ring chunks per wave and step
  static_assert(XT * CPT % 64 == 0 && XT <= 16, "one token tile, whole token segments");
  static_assert(FULL_AFTER < 63, "vmcnt");
  __shared__ MoeRouting rt;
  __shared__ float slot_scale[kMoeMaxPairs + 1];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int P = p.M * p.topk;
  build_routing(rt, p.ids, nullptr, P, p.E);
  const int Ds = uniform(rt.D);
  // every slot's scale, read before the ring (a load inside it would be a
  // vector load: the kernel's own stores may alias alpha for all the
  // compiler knows)
  for (int s = tid; s <= Ds; s += blockDim.x) slot_scale[s] = s < Ds ? p.alpha[rt.expert[s]] : *p.gssh;
  __syncthreads();
  const int tiles_r = (p.I + 127) / 128 * 8;
  const int tiles_s = (p.SI + 127) / 128 * 8;
  // the shared expert's units are (tile, group of XT tokens), so that its
  // M tokens spread over as many waves as a routed expert's few
  const int groups_s = (p.M + XT - 1) / XT;
  const int units = Ds * tiles_r + tiles_s * groups_s;
  const int nsteps = (p.H + 127) / 128;
  const uint32_t row_bytes = static_cast<uint32_t>(p.H) / 2;
  const uint32_t tiles64 = static_cast<uint32_t>(p.H) / 64;
  const rsrc_t rx = make_rsrc(p.x, static_cast<uint32_t>(p.M) * p.H * 2);
  const int stride = gridDim.x * W;

  // chunk of the lane's staging loads (its ring position is lane % CPT)
  uint32_t skc[LX];
#pragma unroll
  for (int i = 0; i < LX; ++i) skc[i] = static_cast<uint32_t>(xl_pos<CPT>(i * (64 / CPT) + lane / CPT, lane % CPT)) * 8;

  // the issue cursor and the per-lane state of its (unit, group)
  MoeJob cur;
  int64_t rows[NA];
  bool rv[NA];
  uint32_t sxo[LX];
  rsrc_t rw = make_rsrc(p.w1, 0), rs = make_rsrc(p.w1s, 0);
  auto load_unit = [&](int u) {
    cur.unit = u < units ? u : -1;
    cur.g0 = 0;
    cur.step = 0;
    cur.nsteps = nsteps;
    if (cur.unit < 0) return;
    const bool shared = u >= Ds * tiles_r;
    const int us = u - Ds * tiles_r;  // shared unit: tile us % tiles_s, group us / tiles_s
    cur.slot = shared ? Ds : u / tiles_r;
    cur.tile = shared ? us % tiles_s : u - cur.slot * tiles_r;
    const int e = shared ? 0 : uniform(static_cast<int>(lds_read_u32(&rt.expert[cur.slot])));
    if (shared) cur.g0 = us / tiles_s * XT;
    cur.cnt = shared ? (cur.g0 + XT < p.M ? cur.g0 + XT : p.M)
                     : uniform(static_cast<int>(lds_read_u32(&rt.count[cur.slot])));
    cur.first = shared ? 0 : uniform(static_cast<int>(lds_read_u32(&rt.start[cur.slot])));
    cur.scale = __builtin_bit_cast(float, uniform(static_cast<int>(lds_read_u32(&slot_scale[cur.slot]))));
    const int half = shared ? p.SI : p.I;
    rw = uniform_rsrc(shared ? p.wsh : p.w1 + e * p.w1_expert_bytes,
                      static_cast<uint32_t>(shared ? p.wsh_bytes : p.w1_expert_bytes));
    rs = uniform_rsrc(shared ? p.ssh : p.w1s + e * p.s1_expert_bytes,
                      static_cast<uint32_t>(shared ? p.ssh_bytes : p.s1_expert_bytes));
    rows[0] = mfma_row<true>(cur.tile, r);
    rv[0] = rows[0] < half;
    rows[1] = rows[0] + half;
    rv[1] = rv[0];
  };
  auto load_group = [&]() {
#pragma unroll
    for (int i = 0; i < LX; ++i) {
      const int idx = cur.g0 + i * (64 / CPT) + lane / CPT;
      const bool ok = cur.unit >= 0 && idx < cur.cnt;
      const bool shared = cur.slot == Ds;
      const int t = shared ? idx : static_cast<int>(lds_read_u32(&rt.order[cur.first + (ok ? idx : 0)])) / p.topk;
      sxo[i] = off_if(ok, static_cast<uint32_t>(t) * p.H * 2);
    }
  };

  u32x4 wb[D][NA];
  uint32_t sb[D][NA];
  MoeJob held[D];
  auto issue = [&](int d) {
    const bool valid = cur.unit >= 0;
    const uint32_t kb = static_cast<uint32_t>(cur.step) * 128;
#pragma unroll
    for (int i = 0; i < LX; ++i) {
      const uint32_t k = kb + skc[i];
      bload16_lds(rx, xl_slot<W * SLOT>(d) + wave * SLOT + i * 64,
                  off_if(valid && k < static_cast<uint32_t>(p.H), sxo[i] + k * 2));
    }
    const uint32_t k = kb + g * 32;
    const bool kv = valid && k < static_cast<uint32_t>(p.H);
#pragma unroll
    for (int a = 0; a < NA; ++a) {
      const bool ok = rv[a] && kv;
      sb[d][a] = bload4(rs, off_if(ok, static_cast<uint32_t>(scale_word_offset(rows[a], k / 64, tiles64))));
      wb[d][a] = bload16_nt(rw, off_if(ok, static_cast<uint32_t>(rows[a]) * row_bytes + k / 2));
    }
    held[d] = cur;
    __builtin_amdgcn_sched_barrier(0);
    if (valid && moe_job_next<XT>(cur)) {
      load_unit(cur.unit + stride);
      load_group();
    } else if (valid && cur.step == 0) {
      load_group();
    }
  };

  f32x4 acc[NA];
  auto finish = [&](const MoeJob& j) {
    const bool shared = j.slot == Ds;
    const int half = shared ? p.SI : p.I;
    const int idx = j.g0 + (lane & 15);
    if ((lane & 15) < XT && idx < j.cnt) {
      const int pair = shared ? 0 : static_cast<int>(lds_read_u32(&rt.order[j.first + idx]));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t row = mfma_row<true>(j.tile, 4 * (lane >> 4) + i);
        if (row >= half) continue;
        float gv = acc[0][i] * j.scale, uv = acc[1][i] * j.scale;
        if (shared) {
          gv = bf16_bits_to_f32(f32_to_bf16_bits(gv));
          uv = bf16_bits_to_f32(f32_to_bf16_bits(uv));
          p.sact[static_cast<int64_t>(idx) * p.SI + row] = f32_to_bf16_bits(silu_f32(gv) * uv);
        } else {
          p.act[static_cast<int64_t>(pair) * p.I + row] = f32_to_bf16_bits(silu_f32(gv) * uv);
        }
      }
    }
  };
  auto consume = [&](int d, int after) {
    vm_wait_n(after);
    u32x4 xf[4];
    const int t = r & (XT - 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) xf[j] = xl_slot<W * SLOT>(d)[wave * SLOT + t * CPT + xl_pos<CPT>(t, 4 * g + j)];
    if (held[d].step == 0) {
#pragma unroll
      for (int a = 0; a < NA; ++a) acc[a] = f32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int a = 0; a < NA; ++a) acc[a] = mfma_16x16x32(fp4_a_fragment(wb[d][a], sb[d][a], g, j), xf[j], acc[a]);
    if (held[d].unit >= 0 && held[d].step == held[d].nsteps - 1) finish(held[d]);
  };

  load_unit(blockIdx.x * W + wave);
  load_group();
#pragma unroll
  for (int d = 0; d < D; ++d) issue(d);
  while (cur.unit >= 0) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      consume(d, FULL_AFTER);
      lds_wait();  // the slot's fragment reads retire before it is refilled
      issue(d);
    }
  }
#pragma unroll
  for (int d = 0; d < D; ++d) consume(d, NA * PER + (D - 1 - d) * L);
}

// down_combine.  A workgroup per 16-row tile of H; its waves take the slots
// round robin (slot D being the shared expert) and run each slot's K (I or
// SI) through their ring, so a slot's job stream is one unit per token
// group.  For every pair the wave forms y = bf16(FP32 sum * alpha2[e]) and
// adds tw * y to its own FP32 partial of the pair's token in LDS, one token
// column at a time (two pairs of a group may share a token); the shared
// expert's y goes to its own LDS rows.  The four partials are added in wave
// order, then out = bf16(bf16(sum) + y_shared).
template <int XT>
__global__ __launch_bounds__(kMoeDownWaves * 64) void k_moe_down_mfma(const MoeDownParams p) {
  constexpr int W = kMoeDownWaves, D = kMoeDownRing, NA = 1, CPT = 16, LX = XT * CPT / 64, PER = 2;
  constexpr int L = LX + NA * PER;
  constexpr int FULL_AFTER = NA * PER + (D - 1) * L;
  constexpr int SLOT = XT * CPT;
  static_assert(XT * CPT % 64 == 0 && XT <= 16, "one token tile, whole token segments");
  static_assert(FULL_AFTER < 63, "vmcnt");
  __shared__ MoeRouting rt;
  __shared__ float part[W][kMoeMaxTokens][16];
  __shared__ float ysh[kMoeMaxTokens][16];
  __shared__ float slot_scale[kMoeMaxPairs + 1];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int P = p.M * p.topk;
  build_routing(rt, p.ids, p.tw, P, p.E);
  const int Ds = uniform(rt.D);
  for (int s = tid; s <= Ds; s += blockDim.x) slot_scale[s] = s < Ds ? p.alpha2[rt.expert[s]] : *p.gssd;
  __syncthreads();
  const int tiles = (p.H + 127) / 128 * 8;
  // Fields chosen per slot, read once into registers.  A choice between two
  // fields of the parameter block would otherwise become one load from a
  // chosen address, i.e. a copy of the block in scratch memory.
  const uint32_t k_routed = static_cast<uint32_t>(uniform(p.I)), k_shared = static_cast<uint32_t>(uniform(p.SI));
  const uint32_t act_bytes = static_cast<uint32_t>(P) * k_routed * 2;
  const uint32_t sact_bytes = static_cast<uint32_t>(p.M) * k_shared * 2;
  const int groups_s = (p.M + XT - 1) / XT;
  const uint8_t* const w2 = uniform_ptr(p.w2);
  const uint8_t* const w2s = uniform_ptr(p.w2s);
  const uint8_t* const wsd = uniform_ptr(p.wsd);
  const uint8_t* const ssd = uniform_ptr(p.ssd);
  const void* const act = uniform_ptr(p.act);
  const void* const sact = uniform_ptr(p.sact);
  const int64_t w2_expert_bytes = uniform_i64(p.w2_expert_bytes), s2_expert_bytes = uniform_i64(p.s2_expert_bytes);
  const uint32_t wsd_bytes = static_cast<uint32_t>(uniform(static_cast<int>(p.wsd_bytes)));
  const uint32_t ssd_bytes = static_cast<uint32_t>(uniform(static_cast<int>(p.ssd_bytes)));

  uint32_t skc[LX];
#pragma unroll
  for (int i = 0; i < LX; ++i) skc[i] = static_cast<uint32_t>(xl_pos<CPT>(i * (64 / CPT) + lane / CPT, lane % CPT)) * 8;

  for (int tile = xcd_logical_block(); tile < tiles; tile += gridDim.x) {
    for (int i = tid; i < W * kMoeMaxTokens * 16; i += blockDim.x) (&part[0][0][0])[i] = 0.0f;
    for (int i = tid; i < kMoeMaxTokens * 16; i += blockDim.x) (&ysh[0][0])[i] = 0.0f;
    __syncthreads();

    MoeJob cur;
    const int64_t row = mfma_row<true>(tile, r);
    const bool rvalid = row < p.H;
    uint32_t sxo[LX];
    // Slots Ds .. Ds + groups_s - 1 are the shared expert's groups of XT
    // tokens (cur.slot is then Ds), so that its M tokens spread over waves.
    auto load_unit = [&](int s) {
      cur.unit = s < Ds + groups_s ? s : -1;
      cur.tile = tile;
      cur.g0 = 0;
      cur.step = 0;
      if (cur.unit < 0) return;
      const bool shared = s >= Ds;
      cur.slot = shared ? Ds : s;
      if (shared) cur.g0 = (s - Ds) * XT;
      cur.expert = shared ? 0 : uniform(static_cast<int>(lds_read_u32(&rt.expert[s])));
      cur.cnt = shared ? (cur.g0 + XT < p.M ? cur.g0 + XT : p.M)
                       : uniform(static_cast<int>(lds_read_u32(&rt.count[s])));
      cur.first = shared ? 0 : uniform(static_cast<int>(lds_read_u32(&rt.start[s])));
      cur.scale = __builtin_bit_cast(float, uniform(static_cast<int>(lds_read_u32(&slot_scale[cur.slot]))));
      cur.nsteps = static_cast<int>((pick(shared, k_shared, k_routed) + 127) / 128);
    };
    auto load_group = [&]() {
      const bool shared = cur.slot == Ds;
      const uint32_t kdim = pick(shared, k_shared, k_routed);
#pragma unroll
      for (int i = 0; i < LX; ++i) {
        const int idx = cur.g0 + i * (64 / CPT) + lane / CPT;
        const bool ok = cur.unit >= 0 && idx < cur.cnt;
        const int xr = shared ? idx : static_cast<int>(lds_read_u32(&rt.order[cur.first + (ok ? idx : 0)]));  // token (shared) or pair row
        sxo[i] = off_if(ok, static_cast<uint32_t>(xr) * kdim * 2);
      }
    };

    u32x4 wb[D];
    uint32_t sb[D];
    MoeJob held[D];
    auto issue = [&](int d) {
      const bool valid = cur.unit >= 0;
      const bool shared = cur.slot == Ds;
      const uint32_t kdim = pick(shared, k_shared, k_routed);
      const int64_t e = cur.expert;
      const rsrc_t rw = uniform_rsrc(pick(shared, wsd, w2 + e * w2_expert_bytes),
                                     pick(shared, wsd_bytes, static_cast<uint32_t>(w2_expert_bytes)));
      const rsrc_t rs = uniform_rsrc(pick(shared, ssd, w2s + e * s2_expert_bytes),
                                     pick(shared, ssd_bytes, static_cast<uint32_t>(s2_expert_bytes)));
      const rsrc_t rx = uniform_rsrc(pick(shared, sact, act), pick(shared, sact_bytes, act_bytes));
      const uint32_t kb = static_cast<uint32_t>(cur.step) * 128;
#pragma unroll
      for (int i = 0; i < LX; ++i) {
        const uint32_t k = kb + skc[i];
        bload16_lds(rx, xl_slot<W * SLOT>(d) + wave * SLOT + i * 64, off_if(valid && k < kdim, sxo[i] + k * 2));
      }
      const uint32_t k = kb + g * 32;
      const bool ok = valid && rvalid && k < kdim;
      sb[d] = bload4(rs, off_if(ok, static_cast<uint32_t>(scale_word_offset(row, k / 64, kdim / 64))));
      wb[d] = bload16_nt(rw, off_if(ok, static_cast<uint32_t>(row) * (kdim / 2) + k / 2));
      held[d] = cur;
      __builtin_amdgcn_sched_barrier(0);
      if (valid && moe_job_next<XT>(cur)) {
        load_unit(cur.unit + W);
        load_group();
      } else if (valid && cur.step == 0) {
        load_group();
      }
    };

    f32x4 acc;
    auto finish = [&](const MoeJob& j) {
      const bool shared = j.slot == Ds;
      const int c = lane & 15;
      const int idx = j.g0 + c;
      const bool has = c < XT && idx < j.cnt;
      const int pair = has && !shared ? static_cast<int>(lds_read_u32(&rt.order[j.first + idx])) : 0;
      float y[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] = bf16_bits_to_f32(f32_to_bf16_bits(acc[i] * j.scale));
      if (shared) {
        if (has) {
#pragma unroll
          for (int i = 0; i < 4; ++i) lds_store_f32(&ysh[idx][4 * (lane >> 4) + i], y[i]);
        }
        return;
      }
      const float w = has ? __builtin_bit_cast(float, lds_read_u32(&rt.tw[pair])) : 0.0f;
      const int tok = pair / p.topk;
      // one token column at a time: two pairs of one group may share a token
      for (int cc = 0; cc < XT; ++cc) {
        if (has && c == cc) {
#pragma unroll
          for (int i = 0; i < 4; ++i) lds_add_f32(&part[wave][tok][4 * (lane >> 4) + i], w * y[i]);
        }
      }
    };
    auto consume = [&](int d, int after) {
      vm_wait_n(after);
      u32x4 xf[4];
      const int t = r & (XT - 1);
#pragma unroll
      for (int j = 0; j < 4; ++j) xf[j] = xl_slot<W * SLOT>(d)[wave * SLOT + t * CPT + xl_pos<CPT>(t, 4 * g + j)];
      if (held[d].step == 0) acc = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = mfma_16x16x32(fp4_a_fragment(wb[d], sb[d], g, j), xf[j], acc);
      if (held[d].unit >= 0 && held[d].step == held[d].nsteps - 1) finish(held[d]);
    };

    load_unit(wave);
    load_group();
#pragma unroll
    for (int d = 0; d < D; ++d) issue(d);
    while (cur.unit >= 0) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        consume(d, FULL_AFTER);
        lds_wait();
        issue(d);
      }
    }
#pragma unroll
    for (int d = 0; d < D; ++d) consume(d, NA * PER + (D - 1 - d) * L);
    lds_wait();  // the partial and shared-expert updates above are not visible to the compiler
    __syncthreads();
    for (int i = tid; i < p.M * 16; i += blockDim.x) {
      const int t = i >> 4, rr = i & 15;
      const int64_t orow = mfma_row<true>(tile, rr);
      if (orow < p.H) {
        float s = part[0][t][rr];
#pragma unroll
        for (int w = 1; w < W; ++w) s += part[w][t][rr];  // wave order
        const float sr = bf16_bits_to_f32(f32_to_bf16_bits(s));
        p.out[static_cast<int64_t>(t) * p.H + orow] = f32_to_bf16_bits(sr + ysh[t][rr]);
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ launch
namespace {

// Persistent gate_up workgroups: about five resident per CU.
constexpr int64_t kMoeGateUpGrid = 1280;
// Persistent MFMA gate_up workgroups: two per CU.
constexpr int64_t kMoeMfmaGrid = 512;

// The MFMA forms from three tokens up; one or two tokens keep the VALU
// forms, whose per-token dot products then cost no more than the MFMA path's
// dequant (measured on the 128-expert decode block).
bool moe_use_mfma(int M) { return M >= 3; }

template <int MT>
hipError_t launch_gate_up_mt(const MoeGateUpParams& p, int c, hipStream_t stream) {
  const int64_t max_items = static_cast<int64_t>(p.slots_max) * ((p.I + 127) / 128 * 32) + (p.SI + 127) / 128 * 32;
  const dim3 grid(static_cast<unsigned>(max_items < kMoeGateUpGrid ? max_items : kMoeGateUpGrid)), block(256);
  switch (c) {
    case 1: hipLaunchKernelGGL((k_moe_gate_up<MT, 1>), grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL((k_moe_gate_up<MT, 2>), grid, block, 0, stream, p); break;
  }
  return hipGetLastError();
}

// Waves per down_combine workgroup (each takes every kMoeDownValuWaves-th slot).
constexpr int kMoeDownValuWaves = 4;

template <int MT>
hipError_t launch_down_mt(const MoeDownParams& p, int c, hipStream_t stream) {
  constexpr int NW = kMoeDownValuWaves;
  const int64_t units = (p.H + 127) / 128 * 32;
  const dim3 grid(static_cast<unsigned>(units < 4096 ? units : 4096)), block(NW * 64);
  switch (c) {
    case 1: hipLaunchKernelGGL((k_moe_down_combine<MT, 1, NW>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((k_moe_down_combine<MT, 2, NW>), grid, block, 0, stream, p); break;
    case 3: hipLaunchKernelGGL((k_moe_down_combine<MT, 3, NW>), grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL((k_moe_down_combine<MT, 4, NW>), grid, block, 0, stream, p); break;
  }
  return hipGetLastError();
}

// Chunk positions per lane: enough to cover K in one block where that fits
// in `cmax`, else `cmax` and several K blocks.
int chunks_per_lane(int64_t k, int64_t lanes, int cmax) {
  const int64_t need = (k / 8 + lanes - 1) / lanes;
  if (need <= 1) return 1;
  if (need <= 2) return 2;
  if (need <= 3 && cmax >= 3) return 3;
  return cmax;
}

}  // namespace

hipError_t launch_moe_gate_up(MoeGateUpParams p, hipStream_t stream) {
  const int pairs = p.M * p.topk;
  p.slots_max = pairs < p.E ? pairs : p.E;
  // (the VALU forms read a quad's scale words as one 16-byte chunk, and
  // route at most kMoeValuMaxPairs pairs)
  if (moe_use_mfma(p.M) || !p.scales16 || pairs > kMoeValuMaxPairs) {
    // one work unit per wave at least, two resident workgroups per CU at most
    const int64_t units = static_cast<int64_t>(p.slots_max) * ((p.I + 127) / 128 * 8) + (p.SI + 127) / 128 * 8;
    int64_t blocks = (units + kMoeGateUpWaves - 1) / kMoeGateUpWaves;
    if (blocks > kMoeMfmaGrid) blocks = kMoeMfmaGrid;
    const dim3 grid(static_cast<unsigned>(blocks)), block(kMoeGateUpWaves * 64);
    if (p.M <= 4) hipLaunchKernelGGL((k_moe_gate_up_mfma<4>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((k_moe_gate_up_mfma<8>), grid, block, 0, stream, p);
    return hipGetLastError();
  }
  const int c = chunks_per_lane(p.H, 4 * 64, 2);
  if (p.M <= 1) return launch_gate_up_mt<1>(p, c, stream);
  return launch_gate_up_mt<2>(p, c, stream);
}

hipError_t launch_moe_down_combine(MoeDownParams p, hipStream_t stream) {
  if (moe_use_mfma(p.M) || !p.scales16 || p.M * p.topk > kMoeValuMaxPairs) {
    const int64_t tiles = (p.H + 127) / 128 * 8;
    const dim3 grid(static_cast<unsigned>(tiles < 4096 ? tiles : 4096)), block(kMoeDownWaves * 64);
    if (p.M <= 4) hipLaunchKernelGGL((k_moe_down_mfma<4>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((k_moe_down_mfma<8>), grid, block, 0, stream, p);
    return hipGetLastError();
  }
  const int64_t kmax = p.I > p.SI ? p.I : p.SI;
  const int c = chunks_per_lane(kmax, 64, 4);
  return launch_down_mt<1>(p, c, stream);
}

}  // namespace w4a16
