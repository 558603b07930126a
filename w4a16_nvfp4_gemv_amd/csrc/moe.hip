// Expert-indexed MoE decode pair (moe_gemv page, module docstring and the
// gate_up / down_combine docstrings).
//
//   gate_up routed: act[p][i] = bf16(silu(g) * u),  g, u = FP32 sum * alpha[e]
//   gate_up shared: sact[t][i] = bf16(silu(bf16(g)) * bf16(u)),  g, u = FP32 sum * gssh
//   down_combine:   y = bf16(FP32 sum * alpha2[e]) per pair,
//                   out = bf16(bf16(sum of tw * y) + y_shared)
//
// Two forms of each kernel:
//
// VALU forms (gate_up up to 8 tokens, down_combine up to 4).  One job per
// pair: a job reads the weights of its pair's expert (two pairs routed to one
// expert read them twice, the second time mostly from L2), so no routing
// table is built and a workgroup needs only the ids of its jobs.
// Chunk-interleaved loads and per-token dot products (chunk_core.hpp).
// gate_up gives every (token, shared-expert quad) and (pair, routed quad)
// item a workgroup whose four waves split H; down_combine gives a workgroup
// a quad of H rows and puts the loads of up to 9 jobs in flight at once.
//
// MFMA forms (above those token counts), expert-major: every routed expert's weights are read
// once per call, for all the tokens routed to it.  Every workgroup rebuilds
// the call's routing in LDS from ids (at most 32 tokens x 16 slots = 512
// pairs): the distinct experts in order of first appearance ("slots"), and
// the pairs of every slot in ascending pair order.  No host synchronization
// and no workspace are needed, and the order of every floating-point sum
// depends on ids alone.  The swap-AB MFMA building blocks of the dense GEMV
// (mfma_core.hpp) take each slot's tokens, gathered by the loads that stage
// activations in LDS; the dequant then costs the same for any number of
// tokens.  Each wave streams whole work units through one LDS ring (see the
// section below).
//
// Inside every ring the loads are counted: no other vector memory access may
// fall between them, and LDS tables are read with lds_read_u32 so that the
// compiler adds no wait for the loads still writing ring slots.
#include <type_traits>

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

// Tokens the VALU forms (one job per pair) take, measured on the 128-expert
// decode block against the MFMA forms (us):
//   gate_up       4 / 6 / 8 tokens 47.2 / 66.8 / 87.3 against 55.0 / 77.0 /
//                 94.8; 16 / 32 tokens 172 / 337 against 152 / 209
//   down_combine  3 / 4 tokens 25.1 / 32.3 against 27.3 / 32.0; 6 / 8 tokens
//                 47.3 / 61.4 against 43.6 / 54.5
constexpr int kMoeGateUpPairsMaxTokens = 8;
constexpr int kMoeDownPairsMaxTokens = 4;
// down_combine keeps one pair per lane of a wave
constexpr int kMoeDownPairsMaxPairs = 64;

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

// ------------------------------------------------------------------ gate_up, one job per pair
// Up to kMoeGateUpPairsMaxTokens tokens: every item is one token's product
// with one quad of gate rows and the matching up rows -- (token t, quad of
// the shared expert's SI rows) first, since they need no id, then (pair j,
// quad of I rows), unit-major, so that the pairs routed to one expert read
// the same rows at about the same time and all but the first read them from
// L2.  A workgroup needs only the id of its item's pair, read by one
// scalar-uniform load, and no routing table.  The 4 waves split H with the
// chunked VALU core (one token per item: the registers of more tokens cost
// more waves per SIMD than the shared reads save).
template <int C>
__global__ __launch_bounds__(256) void k_moe_gate_up_pairs(const MoeGateUpParams p) {
  constexpr int KS = 4;                 // waves per item, each a slice of H
  constexpr int PV = 2;                 // gate, up
  constexpr int V = 4 * PV;             // value index q * 2 + w
  using RS = ReduceScatter<V, PV>;
  __shared__ float red[KS - 1][RS::LEFT][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int kw = uniform(tid >> 6);
  const int P = p.M * p.topk;
  const int units_r = (p.I + 127) / 128 * 32;
  const int units_s = (p.SI + 127) / 128 * 32;
  const int items_s = p.M * units_s;
  const uint32_t nch = p.H / 8;
  const int nkb = static_cast<int>((nch + KS * C * 64 - 1) / (KS * C * 64));
  const uint32_t shift = 8u * ((lane >> 1) & 3);
  const uint32_t row_bytes = p.H / 2;
  const uint32_t tiles = p.H / 64;
  const rsrc_t rx = make_rsrc(p.x, static_cast<uint32_t>(p.M) * p.H * 2);
  const float gssh = *p.gssh;

  // t: the item's token; j: its pair (routed items).  UPQ: the up rows form
  // aligned quads too (rows of an expert a multiple of 128), so the scale
  // loads need no branch (as a runtime branch it split the loads, and the
  // compiler waited for some of them before issuing the rest)
  auto run = [&](auto upq_tag, bool shared, int t, int j, int u) {
    constexpr bool UPQ = decltype(upq_tag)::value;
    const int half = shared ? p.SI : p.I;
    int64_t rows[8];
    bool rv[8];
    quad_rows<8>(u, half, half, rows, rv);
    const bool quad_ok[2] = {true, UPQ};
    const uint32_t xoff[1] = {static_cast<uint32_t>(t) * p.H * 2};
    float acc[8][1];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i][0] = 0.0f;
    const int e = shared ? 0 : clamp_expert(uniform(p.ids[j]), p.E);
    const float scale = shared ? gssh : p.alpha[e];
    const rsrc_t rw = uniform_rsrc(shared ? p.wsh : p.w1 + e * p.w1_expert_bytes,
                                   static_cast<uint32_t>(shared ? p.wsh_bytes : p.w1_expert_bytes));
    const rsrc_t rs = uniform_rsrc(shared ? p.ssh : p.w1s + e * p.s1_expert_bytes,
                                   static_cast<uint32_t>(shared ? p.ssh_bytes : p.s1_expert_bytes));
    for (int kb = 0; kb < nkb; ++kb) {
      uint32_t ch[C];
      bool ok[C];
#pragma unroll
      for (int q = 0; q < C; ++q) {
        ch[q] = static_cast<uint32_t>((kb * KS + kw) * C + q) * 64 + lane;
        ok[q] = ch[q] < nch;
      }
      ChunkX<C, 1> xb;
      ChunkW<C, 8> wb;
      chunk_issue_x<C, 1>(xb, rx, xoff, ch, ok);
      chunk_issue_w<C, 8>(wb, rw, row_bytes, rs, tiles, rows, rv, quad_ok, ch, ok);
      __builtin_amdgcn_sched_barrier(0);  // every load ahead of the arithmetic
      chunk_compute<C, 8, 1>(wb, xb, shift, acc);
    }
    float v[V];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int w = 0; w < PV; ++w) v[q * PV + w] = acc[4 * w + q][0];
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
        const int q = (base + i * PV) / PV;
        const int64_t row = static_cast<int64_t>(u >> 5) * 128 + (u & 31) + 32 * q;
        if ((lane & 15) == i && row < half) {
          float g = v[i * PV] * scale, up = v[i * PV + 1] * scale;
          if (shared) {
            g = bf16_bits_to_f32(f32_to_bf16_bits(g));
            up = bf16_bits_to_f32(f32_to_bf16_bits(up));
            p.sact[static_cast<int64_t>(t) * p.SI + row] = f32_to_bf16_bits(silu_f32(g) * up);
          } else {
            p.act[static_cast<int64_t>(j) * p.I + row] = f32_to_bf16_bits(silu_f32(g) * up);
          }
        }
      }
    }
    __syncthreads();
  };

  // The grid is exactly one workgroup per item, so no loop or range check
  // stands between the kernel arguments and the first loads (with a loop
  // over items, the expert id's load waited behind the loop's entry test:
  // 0.3-0.5 us slower at one token).
  {
    const int item = xcd_logical_block();
    if (item < items_s) {
      const int t = item / units_s;
      const int u = item - t * units_s;
      if (p.SI % 128 == 0) run(std::true_type{}, true, t, 0, u);
      else run(std::false_type{}, true, t, 0, u);
    } else {
      const int u = (item - items_s) / P;
      const int j = item - items_s - u * P;
      if (p.I % 128 == 0) run(std::true_type{}, false, j / p.topk, j, u);
      else run(std::false_type{}, false, j / p.topk, j, u);
    }
  }
}

// ------------------------------------------------------------------ down_combine, one job per pair
// Up to four tokens: the work of a quad of H rows is P + M jobs, the shared
// expert for each token and then every pair in order (pair j reads the
// weights of expert ids[j] and its own act row; two pairs routed to one
// expert read its weights twice, the second time from L2).  No routing table
// is built: a job needs only its pair's id, and the shared jobs, which need
// none, are issued while the ids arrive.  The NW waves split the K of every
// job (lane l of wave w takes chunks (c * NW + w) * 64 + l), so all SG jobs
// of a group are in flight at once; their sums are reduced across the lanes
// and waves, rounded to BF16 (y_j = bf16(acc * alpha2[e_j]), y_shared =
// bf16(acc * gssd)), and the combine adds tw_j * y_j over j in ascending
// order in FP32 before the two BF16 roundings of the moe_gemv page.
constexpr int kMoeDownPairsMaxJobs = kMoeDownPairsMaxPairs + kMoeDownPairsMaxTokens;

template <int NW, int CL, int SG>
__global__ __launch_bounds__(NW * 64) void k_moe_down_pairs(const MoeDownParams p) {
  constexpr int R = 4;       // rows of a workgroup: one quad of H rows
  constexpr int V = SG * R;  // value index job * R + q
  using RS = ReduceScatter<V, 1>;
  __shared__ float red[NW][V];
  __shared__ float yv[kMoeDownPairsMaxJobs][R];  // jobs 0..M-1: shared expert, then pairs
  __shared__ float tws[kMoeDownPairsMaxPairs];
  __shared__ float a2s[kMoeDownPairsMaxPairs];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int P = p.M * p.topk;
  const int J = p.M + P;
  // every pair's id, alpha2 and routing weight, issued first (vector loads:
  // the waits the compiler adds for them come after the shared jobs' loads)
  // (unconditional loads: a branch around them would make the compiler wait
  // for them inside it, before the shared jobs' loads)
  const int my_id = p.ids[lane < P ? lane : 0];
  const float my_tw = p.tw[lane < P ? lane : 0];
  float my_a2 = 0.0f;  // loaded once the first jobs' loads are issued
  const float gssd = *p.gssd;
  const int64_t units = (p.H + 127) / 128 * 32;
  const uint32_t shift = 8u * ((lane >> 1) & 3);
  const uint32_t act_bytes = static_cast<uint32_t>(P) * p.I * 2;
  const uint32_t sact_bytes = static_cast<uint32_t>(p.M) * p.SI * 2;
  bool tw_stored = false;

  // At most one workgroup per unit, so the first unit is this workgroup's
  // without a test: with the test ahead of the body, the compiler moved the
  // id and routing-weight loads behind it and three waits for kernel
  // arguments (0.2 us at one token).
  int64_t u = xcd_logical_block();
  do {
    int64_t rows[R];
    bool rv[R];
    quad_rows<R>(u, p.H, 0, rows, rv);
    const bool quad_ok[1] = {true};
    for (int g0 = 0; g0 < J; g0 += SG) {
      ChunkW<CL, R> wb[SG];
      ChunkX<CL, 1> xb[SG];
#pragma unroll
      for (int s = 0; s < SG; ++s) {
        const int j = g0 + s;
        const bool valid = j < J;
        const bool shared = j < p.M;
        const int pair = shared ? 0 : (valid ? j - p.M : 0);
        int e = 0;
        if (!shared) e = clamp_expert(__builtin_amdgcn_readlane(my_id, pair), p.E);  // (no wait for the ids in shared jobs)
        const int k = shared ? p.SI : p.I;
        const uint32_t nch = k / 8;
        uint32_t ch[CL];
        bool ok[CL];
#pragma unroll
        for (int c = 0; c < CL; ++c) {
          ch[c] = static_cast<uint32_t>(c * NW + wave) * 64 + lane;
          ok[c] = valid && ch[c] < nch;
        }
        const uint32_t xoff[1] = {static_cast<uint32_t>(shared ? j : pair) * k * 2};
        chunk_issue_x<CL, 1>(xb[s],
                             uniform_rsrc(shared ? static_cast<const void*>(p.sact) : static_cast<const void*>(p.act),
                                          shared ? sact_bytes : act_bytes),
                             xoff, ch, ok);
        const uint8_t* wbase = shared ? p.wsd : p.w2 + e * p.w2_expert_bytes;
        const uint8_t* sbase = shared ? p.ssd : p.w2s + e * p.s2_expert_bytes;
        const uint32_t wbytes = static_cast<uint32_t>(shared ? p.wsd_bytes : p.w2_expert_bytes);
        const uint32_t sbytes = static_cast<uint32_t>(shared ? p.ssd_bytes : p.s2_expert_bytes);
        chunk_issue_w<CL, R>(wb[s], uniform_rsrc(wbase, wbytes), k / 2, uniform_rsrc(sbase, sbytes), k / 64, rows, rv,
                             quad_ok, ch, ok);
      }
      if (!tw_stored) my_a2 = p.alpha2[clamp_expert(my_id, p.E)];
      __builtin_amdgcn_sched_barrier(0);  // every load of the group ahead of the arithmetic
      float v[V];
#pragma unroll
      for (int s = 0; s < SG; ++s) {
        float acc[R][1];
#pragma unroll
        for (int i = 0; i < R; ++i) acc[i][0] = 0.0f;
        chunk_compute<CL, R, 1>(wb[s], xb[s], shift, acc);
#pragma unroll
        for (int i = 0; i < R; ++i) v[s * R + i] = acc[i][0];
      }
      reduce_scatter<V, 1>(v);
      const int base = reduce_scatter_base<V, 1>(lane);
      if ((lane & 15) == 0) {
#pragma unroll
        for (int i = 0; i < RS::LEFT; ++i) red[wave][base + i] = v[i];
      }
      if (!tw_stored && wave == 0 && lane < P) {
        tws[lane] = my_tw;
        a2s[lane] = my_a2;
      }
      tw_stored = true;
      __syncthreads();
      if (tid < V) {
        const int j = g0 + tid / R;
        if (j < J) {
          float t = red[0][tid];
#pragma unroll
          for (int w = 1; w < NW; ++w) t += red[w][tid];  // in wave order
          const float scale = j < p.M ? gssd : a2s[j - p.M];
          yv[j][tid % R] = bf16_bits_to_f32(f32_to_bf16_bits(t * scale));
        }
      }
      __syncthreads();
    }
    if (tid < p.M * R) {
      const int t = tid / R, q = tid % R;
      if (rv[q]) {
        float acc = 0.0f;
        for (int j = 0; j < p.topk; ++j) acc += tws[t * p.topk + j] * yv[p.M + t * p.topk + j][q];
        const float sr = bf16_bits_to_f32(f32_to_bf16_bits(acc));
        p.out[static_cast<int64_t>(t) * p.H + rows[q]] = f32_to_bf16_bits(sr + yv[t][q]);
      }
    }
    __syncthreads();
    u += gridDim.x;
  } while (u < units);
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
    // staging loads, then weight loads, in the order the waits count them
    __builtin_amdgcn_sched_barrier(0);
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
      // staging loads, then weight loads, in the order the waits count them
      __builtin_amdgcn_sched_barrier(0);
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

// Persistent MFMA gate_up workgroups: two per CU.
constexpr int64_t kMoeMfmaGrid = 512;


// The longest K (I or SI, in 8-k chunks) the one-block VALU down_combine
// takes: 4 waves x 64 lanes x 2 chunks.
constexpr int64_t kMoeDownPairsMaxChunks = 4 * 64 * 2;

template <int NW, int CL, int SG>
hipError_t launch_down_pairs_sg(const MoeDownParams& p, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((k_moe_down_pairs<NW, CL, SG>), grid, dim3(NW * 64), 0, stream, p);
  return hipGetLastError();
}

template <int NW, int CL>
hipError_t launch_down_pairs_cl(const MoeDownParams& p, int sg, dim3 grid, hipStream_t stream) {
  if constexpr (CL == 1) {
    if (sg >= 9) return launch_down_pairs_sg<NW, CL, 9>(p, grid, stream);
    if (sg >= 5) return launch_down_pairs_sg<NW, CL, 5>(p, grid, stream);
  }
  if (sg >= 4) return launch_down_pairs_sg<NW, CL, 4>(p, grid, stream);
  if (sg >= 2) return launch_down_pairs_sg<NW, CL, 2>(p, grid, stream);
  return launch_down_pairs_sg<NW, CL, 1>(p, grid, stream);
}

hipError_t launch_down_pairs(const MoeDownParams& p, int nw, int cl, int sg, dim3 grid, hipStream_t stream) {
  switch (nw * 10 + cl) {
    case 11: return launch_down_pairs_cl<1, 1>(p, sg, grid, stream);
    case 21: return launch_down_pairs_cl<2, 1>(p, sg, grid, stream);
    case 31: return launch_down_pairs_cl<3, 1>(p, sg, grid, stream);
    case 41: return launch_down_pairs_cl<4, 1>(p, sg, grid, stream);
    default: return launch_down_pairs_cl<4, 2>(p, sg, grid, stream);
  }
}

}  // namespace

hipError_t launch_moe_gate_up(MoeGateUpParams p, hipStream_t stream) {
  const int pairs = p.M * p.topk;
  p.slots_max = pairs < p.E ? pairs : p.E;
  // (the VALU form reads a quad's scale words as one 16-byte chunk)
  if (p.M > kMoeGateUpPairsMaxTokens || !p.scales16) {
    // one work unit per wave at least, two resident workgroups per CU at most
    const int64_t units = static_cast<int64_t>(p.slots_max) * ((p.I + 127) / 128 * 8) + (p.SI + 127) / 128 * 8;
    int64_t blocks = (units + kMoeGateUpWaves - 1) / kMoeGateUpWaves;
    if (blocks > kMoeMfmaGrid) blocks = kMoeMfmaGrid;
    const dim3 grid(static_cast<unsigned>(blocks)), block(kMoeGateUpWaves * 64);
    if (p.M <= 4) hipLaunchKernelGGL((k_moe_gate_up_mfma<4>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((k_moe_gate_up_mfma<8>), grid, block, 0, stream, p);
    return hipGetLastError();
  }
  // exactly one item per workgroup, which the kernel relies on (a persistent
  // grid of 1280 or 2560 workgroups measured 1.6 / 3.7 us slower at one
  // token); the 4 waves' 8-k chunks
  // cover H in one block up to 2048 columns with one chunk per lane
  const int64_t items =
      static_cast<int64_t>(pairs) * ((p.I + 127) / 128 * 32) + static_cast<int64_t>(p.M) * ((p.SI + 127) / 128 * 32);
  const dim3 grid(static_cast<unsigned>(items)), block(256);
  if (p.H / 8 <= 4 * 64) hipLaunchKernelGGL((k_moe_gate_up_pairs<1>), grid, block, 0, stream, p);
  else hipLaunchKernelGGL((k_moe_gate_up_pairs<2>), grid, block, 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_moe_down_combine(MoeDownParams p, hipStream_t stream) {
  const int64_t nch = (p.I > p.SI ? p.I : p.SI) / 8;
  // (rows of I or SI beyond kMoeDownPairsMaxChunks chunks also take the
  // MFMA form, which runs any K)
  if (p.M > kMoeDownPairsMaxTokens || !p.scales16 || p.M * p.topk > kMoeDownPairsMaxPairs ||
      nch > kMoeDownPairsMaxChunks) {
    const int64_t tiles = (p.H + 127) / 128 * 8;
    const dim3 grid(static_cast<unsigned>(tiles < 4096 ? tiles : 4096)), block(kMoeDownWaves * 64);
    if (p.M <= 4) hipLaunchKernelGGL((k_moe_down_mfma<4>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((k_moe_down_mfma<8>), grid, block, 0, stream, p);
    return hipGetLastError();
  }
  // waves and chunks per lane that cover the longer K in one block; SG jobs
  // in flight at once, SG * CL * 6 loads (+3) within vmcnt's 63
  const int nw = static_cast<int>(nch <= 64 ? 1 : nch <= 128 ? 2 : nch <= 192 ? 3 : 4);
  const int cl = nch <= nw * 64 ? 1 : 2;
  const int jobs = p.M + p.M * p.topk;
  const int sg_max = cl == 1 ? 9 : 4;
  const int sg = jobs < sg_max ? jobs : sg_max;
  const int64_t units = (p.H + 127) / 128 * 32;
  const dim3 grid(static_cast<unsigned>(units < 8192 ? units : 8192));  // never more than units
  return launch_down_pairs(p, nw, cl, sg, grid, stream);
}

}  // namespace w4a16
