// Paged decode attention for gfx950: one query token per sequence attends over
// the K/V rows its block table names (page "vLLM推理引擎深度解析" §五,
// PagedAttention.forward: per sequence look up the block table, read K and V
// from the physical blocks in place, score q·k/sqrt(d), softmax, weight V).
//
// Work mapping (one workgroup = one (sequence, kv head), or one token partition
// of it in the split-KV variant; its W waves take the blocks round-robin, so
// every wave of a long sequence has the same number of blocks to walk; grid
// rows take the sequences longest first):
//   * A token row of one head is D*e bytes (256 B for 16-bit D=128 or fp32 D=64).
//     LPR = D*e/16 lanes cover a row with one 16-byte load each; a wave covers
//     ROWS = 64/LPR rows per load, so a 16-token block is TPL = 16/ROWS loads of
//     K and TPL of V per lane, each 16-byte and each row segment fully used.
//   * The G query heads of the group share every K/V row: each lane keeps its
//     16-byte slice of all G query vectors in registers and forms G partial dot
//     products per row (packed dot2 for 16-bit types).
//   * Reduce-scatter instead of G all-reductions: the G partials of a row are
//     summed over the row's LPR lanes with a DPP butterfly in which every stage
//     keeps half of the heads and hands the other half to the partner lane, so
//     the G full sums cost G-1 exchanges (plus the plain stages once one head is
//     left) instead of G*log2(LPR). Afterwards lane c of a row owns the score of
//     one head, owner(c); the lane order of the heads is a fixed linear (XOR)
//     map of c chosen so that every DPP partner pattern lines up. Softmax
//     bookkeeping (one exp, one running sum) is then done once per (token, head)
//     instead of once per lane, and an all-gather through the same butterfly
//     hands every lane the G probabilities it needs for its P·V columns.
//   * Online softmax with a wave-uniform reference max per head: scores are in
//     log2 units (scale*log2 e folded in), p = 2^(s - m_ref). m_ref only moves
//     when some score exceeds it by more than 8 (ballot, uniform branch), which
//     bounds p by 256 and makes the rescale of the accumulators rare. The
//     softmax is unchanged by the choice of reference, which cancels in o/l.
//   * Every lane accumulates p*V for its own columns and tokens; rows are
//     summed once at the end, then waves are merged through LDS with the usual
//     max-rescale.
//   * Masking: only the last block of a sequence can hold dead rows (they may
//     hold stale NaN); their scores become -inf and their V slices are zeroed
//     before use, so 0 * NaN never happens.
//   * Block ids are wave-uniform (scalar loads, read a step ahead); two register
//     buffers keep the next block's K/V loads in flight while a block is computed.
//
// Split-KV: partition p of a sequence covers logical tokens
// [partition_size*p, partition_size*(p+1)); its unnormalised output row and
// (max, normaliser) per query head are merged by log-sum-exp. Three plans,
// chosen by the number of partitions a sequence can have and the cache type:
//   * up to 16 (short and mixed contexts): workgroup items. A workgroup walks
//     one (kv head, sequence, partition) item with its waves taking the
//     blocks round-robin; a one-partition sequence is written directly.
//   * more, 16-bit caches: span items. A workgroup takes W consecutive
//     partitions of one (kv head, sequence), wave w walks the w-th on its
//     own, and the W partials are merged in LDS before one row per head goes
//     to the workspace (a sequence with a single span is written directly).
//   * more, fp8 cache: wave items. Every wave walks one partition on its own
//     and writes its partial straight to the workspace (see split_work).
// A second kernel merges what reached the workspace. Items are handed out by
// a work counter in all three.
#include <math.h>

#include <algorithm>

#include "pa_device.h"
#include "pa_launch.h"


namespace pa {

static_assert(static_cast<int>(DT::FP8) == kKvFp8, "cache type codes agree");

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.0f;   // log2 units: p <= 2^8 between rescales

// ---------------------------------------------------------------------------
// Butterfly over the LPR lanes of a row. Stage S exchanges with partner
// lane c ^ PI_S, PI = {1, 2, 7, 15, 16} (quad perms, half-row mirror, row
// mirror, then a cross-row swap for 32-lane rows).
// ---------------------------------------------------------------------------
template <int S>
__device__ __forceinline__ float xchg(float v) {
  if constexpr (S == 1) return dpp_f<0xB1>(v);
  else if constexpr (S == 2) return dpp_f<0x4E>(v);
  else if constexpr (S == 3) return dpp_f<0x141>(v);
  else if constexpr (S == 4) return dpp_f<0x140>(v);
  else return __shfl_xor(v, 16);
}

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x >> 1); }

// Head owned by lane c of a row after the reduce-scatter. Position i of a
// lane's G-vector holds head i ^ owner(c). Stage S (S <= log2 G) splits n =
// G >> (S-1) values in halves, so the partner's position i + n/2 must name the
// same head as the lane's position i: owner(c ^ PI_S) = owner(c) ^ n/2. Stages
// past log2 G are plain sums and need owner(c ^ PI_S) = owner(c). With owner
// linear over the bits of c (bit b contributes M_b), these conditions fix M.
template <int G>
struct HeadMap {
  static constexpr int mu(int s) { return G >> s; }
  static constexpr int M0 = mu(1);
  static constexpr int M1 = mu(2);
  static constexpr int M2 = mu(3) ^ mu(1) ^ mu(2);
  static constexpr int M3 = mu(4) ^ mu(3);
  static constexpr int M4 = mu(5);
  static __device__ __forceinline__ int owner(int c) {
    return ((c & 1) ? M0 : 0) ^ ((c & 2) ? M1 : 0) ^ ((c & 4) ? M2 : 0) ^ ((c & 8) ? M3 : 0) ^
           ((c & 16) ? M4 : 0);
  }
};

template <int G, int LPR, int S = 1>
__device__ __forceinline__ void reduce_scatter(float* v) {
  if constexpr ((1 << (S - 1)) < LPR) {
    constexpr int n = G >> (S - 1);
    if constexpr (n >= 2) {
#pragma unroll
      for (int i = 0; i < n / 2; ++i) v[i] += xchg<S>(v[i + n / 2]);
    } else {
      v[0] += xchg<S>(v[0]);
    }
    reduce_scatter<G, LPR, S + 1>(v);
  }
}

// Inverse of the scatter stages: from v[0] (the owned head) to all G positions.
template <int G, int S = ilog2(G)>
__device__ __forceinline__ void all_gather(float* v) {
  if constexpr (S >= 1) {
    constexpr int n = G >> (S - 1);
#pragma unroll
    for (int i = n / 2; i < n; ++i) v[i] = xchg<S>(v[i - n / 2]);
    all_gather<G, S - 1>(v);
  }
}

// Dot product of two 16-byte vectors, 16-bit types: the first dot2 of the chain
// is the VOP3P form with an inline zero accumulator, the rest accumulate.
template <DT dt>
__device__ __forceinline__ float dot2_first(uint32_t a, uint32_t b) {
  float r;
  if constexpr (dt == DT::BF16)
    asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  else
    asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

template <DT dt>
__device__ __forceinline__ float dot2_acc(uint32_t a, uint32_t b, float acc) {
  if constexpr (dt == DT::BF16)
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162v, a), __builtin_bit_cast(bf162v, b), acc,
                                          false);
  else
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, a), __builtin_bit_cast(half2v, b), acc, false);
}

template <DT dt>
__device__ __forceinline__ float row_dot(const u32x4& a, const u32x4& b) {
  if constexpr (dt == DT::F32) {
    return dot16<dt>(a, b, 0.f);
  } else {
    const uint32_t a0 = a[0], b0 = b[0], a1 = a[1], b1 = b[1], a2 = a[2], b2 = b[2], a3 = a[3], b3 = b[3];
    float acc = dot2_first<dt>(a0, b0);
    acc = dot2_acc<dt>(a1, b1, acc);
    acc = dot2_acc<dt>(a2, b2, acc);
    return dot2_acc<dt>(a3, b3, acc);
  }
}

// Two fp32 values rounded (to nearest even) into one dword of the 16-bit type.
template <DT dt>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = {lo, hi};
  if constexpr (dt == DT::BF16)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf162v));
  else
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, half2v));
}

// 1.0 in both halves of a dword of the 16-bit type (sum of a packed pair by dot2)
template <DT dt>
constexpr uint32_t kOnes2 = dt == DT::BF16 ? 0x3F803F80u : 0x3C003C00u;

// Longest-first dispatch. Workgroups are launched in grid order and a long
// sequence that starts late leaves the chip idle at the end, so grid row r
// takes the sequence of rank r in descending length (ties by index). Every
// workgroup computes the same ranking: lengths fall into 4 buckets per
// octave, buckets are counted in LDS and an exclusive scan gives each bucket
// its first rank; the members of each bucket are gathered (in any order) and
// a sequence's rank inside its bucket is the number of members with a larger
// key (length, then reversed index) - a pure function of the lengths, so all
// workgroups agree and the rows form a permutation of 0..B-1. Which
// workgroup computes a sequence does not change its result. Batches above
// kRankMaxSeqs sequences keep grid order.
constexpr int kBuckets = 128;
constexpr int kRankMaxSeqs = 1024;
// Up to this many sequences, a thread per sequence counts the larger keys
// directly (two barriers; the same order, since buckets are monotone in
// length and keys break ties the same way) — cheaper than the bucket pass.
constexpr int kRankDirectSeqs = 128;

__device__ __forceinline__ int length_bucket(int L) {
  if (L <= 0) return kBuckets - 1;
  const int e = 31 - __clz(L);                                   // floor(log2 L)
  const int m = (e >= 2 ? (L >> (e - 2)) : (L << (2 - e))) & 3;  // next two bits
  return kBuckets - 1 - min(4 * e + m, kBuckets - 1);            // longer: earlier
}

__device__ __forceinline__ int rank_key(int L, int t) {          // unique for t < 1024
  return (min(max(L, 0), (1 << 21) - 1) << 10) | (1023 - t);
}

template <int NT>
__device__ __forceinline__ int sequence_of_row(const int32_t* lens, int B, int r, int& len) {
  static_assert(NT >= kBuckets / 2, "one scan wave covers the buckets");
  if (B > kRankMaxSeqs) {
    len = lens[r];
    return r;
  }
  if (B <= kRankDirectSeqs && B <= NT) {     // small batch: count larger keys directly
    __shared__ int s_k[kRankDirectSeqs];
    __shared__ int s_pick1, s_len1;
    const int t = threadIdx.x;
    const int Lt = t < B ? lens[t] : 0;
    const int key = rank_key(Lt, t);
    if (t < B) s_k[t] = key;
    __syncthreads();
    if (t < B) {
      int rank = 0;
      for (int u = 0; u < B; ++u) rank += s_k[u] > key;   // every lane reads the same word: a broadcast
      if (rank == r) {
        s_pick1 = t;
        s_len1 = Lt;                           // the length travels with the pick
      }
    }
    __syncthreads();
    len = __builtin_amdgcn_readfirstlane(s_len1);
    return __builtin_amdgcn_readfirstlane(s_pick1);
  }
  __shared__ int s_base[kBuckets];
  __shared__ int s_cur[kBuckets];
  __shared__ int s_key[kRankMaxSeqs];
  __shared__ int s_pick, s_len;
  for (int i = threadIdx.x; i < kBuckets; i += NT) s_cur[i] = 0;
  __syncthreads();
  for (int t = threadIdx.x; t < B; t += NT) atomicAdd(&s_cur[length_bucket(lens[t])], 1);
  __syncthreads();
  if (threadIdx.x < 64) {                                        // exclusive scan, 2 buckets a lane
    const int l = threadIdx.x;
    const int c0 = s_cur[2 * l], c1 = s_cur[2 * l + 1];
    int inc = c0 + c1;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(inc, o);
      if (l >= o) inc += y;
    }
    const int exc = inc - c0 - c1;
    s_base[2 * l] = exc;
    s_base[2 * l + 1] = exc + c0;
    s_cur[2 * l] = exc;
    s_cur[2 * l + 1] = exc + c0;
  }
  __syncthreads();
  for (int t = threadIdx.x; t < B; t += NT) {                    // gather bucket members
    const int L = lens[t];
    s_key[atomicAdd(&s_cur[length_bucket(L)], 1)] = rank_key(L, t);
  }
  __syncthreads();
  for (int t = threadIdx.x; t < B; t += NT) {
    const int L = lens[t];
    const int k = length_bucket(L), key = rank_key(L, t);
    const int lo = s_base[k], hi = s_cur[k];
    int rank = lo;
    for (int j = lo; j < hi; ++j) rank += s_key[j] > key;
    if (rank == r) {
      s_pick = t;
      s_len = L;
    }
  }
  __syncthreads();
  len = __builtin_amdgcn_readfirstlane(s_len);
  return __builtin_amdgcn_readfirstlane(s_pick);
}

// Blocks a split-KV call walks for a sequence of L tokens, at most the
// max_parts planned partitions: a sequence longer than the max_context_len the
// call was planned for (a precondition violation) is cut there rather than
// written past the workspace.
__device__ __forceinline__ int split_blocks(const DecodeParams& p, int L) {
  const int nb = min((max(L, 0) + kBlockSize - 1) / kBlockSize, p.block_table_stride);
  return min(nb, p.max_blocks);
}

// Work units (partitions, or spans of partitions) of a sequence of L tokens.
__device__ __forceinline__ int parts_of(const DecodeParams& p, int L) {
  return (split_blocks(p, L) + p.partition_blocks - 1) / p.partition_blocks;
}

// 64 lanes turn v[0..n) into its exclusive prefix sums in place, v[n] = total.
__device__ __forceinline__ void wave_exclusive_scan(int* v, int n) {
  const int l = threadIdx.x & 63;
  const int per = (n + 63) / 64;
  const int t0 = min(l * per, n), t1 = min(t0 + per, n);
  int run = 0;
  for (int t = t0; t < t1; ++t) run += v[t];
  int inc = run;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(inc, o);
    if (l >= o) inc += y;
  }
  int acc = inc - run;
  for (int t = t0; t < t1; ++t) {
    const int c = v[t];
    v[t] = acc;
    acc += c;
  }
  if (l == 63) v[n] = inc;
}

// Split-KV work assignment. A work item is one (kv head, sequence, partition)
// triple that exists. Workgroups start in grid order, and the compute units
// of the chip do not all finish their share at the same rate (each XCD takes
// every eighth workgroup, and some XCDs run slower than others), so items are
// not bound to grid positions: thread 0 of each workgroup takes W consecutive
// tickets from a work counter (zeroed before the launch) and wave w takes
// ticket t + w. Tickets run over the kv heads fastest, then over the
// (sequence, partition) pairs numbered densely, sequence by sequence and the
// partitions of a sequence in order; the grid carries a quarter more
// workgroups than the largest possible number of items needs, so a slow part
// of the chip simply takes fewer tickets and the spare workgroups find none.
// Every workgroup computes the per-sequence prefix sums of partition counts
// in LDS. Batches above kRankMaxSeqs sequences number all num_seqs *
// max_parts pairs instead, empty ones included.
template <int NT>
__device__ __forceinline__ bool split_work(const DecodeParams& p, int wave, int& g, int& b, int& part) {
  __shared__ int s_pre[kRankMaxSeqs + 1];
  __shared__ int s_ticket;
  const int B = p.num_seqs;
  const bool dense = B <= kRankMaxSeqs;
  if (threadIdx.x == 0) s_ticket = atomicAdd(p.ws_ctr, NT / 64);
  if (dense) {
    for (int t = threadIdx.x; t < B; t += NT) s_pre[t] = parts_of(p, p.context_lens[t]);
  }
  __syncthreads();
  if (dense && threadIdx.x < 64) wave_exclusive_scan(s_pre, B);   // a run of sequences per lane
  __syncthreads();
  // LDS reads at uniform addresses, made visibly uniform so that the search,
  // the exit and everything derived from (g, b, part) stay scalar
  const int ticket = __builtin_amdgcn_readfirstlane(s_ticket) + wave;
  g = ticket % p.num_kv_heads;
  const int item = ticket / p.num_kv_heads;
  if (!dense) {
    b = item / p.max_parts;
    part = item % p.max_parts;
    return b < B;
  }
  if (item >= __builtin_amdgcn_readfirstlane(s_pre[B])) return false;
  int lo = 0, hi = B - 1;                   // last sequence whose first item is <= item
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (__builtin_amdgcn_readfirstlane(s_pre[mid]) <= item) lo = mid; else hi = mid - 1;
  }
  b = lo;
  part = item - __builtin_amdgcn_readfirstlane(s_pre[lo]);
  return true;
}

__global__ void splitkv_reset_kernel(int32_t* ctr) {
  if (threadIdx.x == 0) *ctr = 0;
}

// Split-KV with workgroup items. When every sequence has only a few
// partitions (short and mixed contexts), a partition walked by one wave is too
// little work per wave, while one workgroup per sequence leaves the longest
// sequence running alone at the end. Here one workgroup takes one (kv head,
// sequence, partition) item at a time, its W waves share the partition's
// blocks round-robin as in the single pass, and a sequence with a single
// partition writes its output directly (only longer ones go through the
// workspace and the merge). Workgroups are persistent: each takes items from
// the work counter until none is left, so the grid only has to fill the chip.
// Items are numbered kv head fastest, then sequence by sequence in descending
// length (the ranking of the single pass) and partition by partition, so the
// largest items are taken first and the last ones are the shortest. Every
// workgroup builds that numbering once in LDS: the rank order perm[] and the
// exclusive prefix sums pre[] of the partition counts in rank order. Batches
// above kRankMaxSeqs sequences number all num_seqs * max_parts pairs in
// sequence order instead (empty pairs are skipped).
enum : int { kSingle = 0, kWaveItems = 1, kGroupItems = 2, kSpanItems = 3 };
constexpr int kPlanCur = kBuckets;                       // [0, kBuckets): bucket bases
constexpr int kPlanPre = 2 * kBuckets;                   // bucket members, then pre[0..B]
constexpr int kPlanPerm = kPlanPre + kRankMaxSeqs + 1;   // perm[rank] = sequence
constexpr int kPlanTicket = kPlanPerm + kRankMaxSeqs;
constexpr int kPlanInts = kPlanTicket + 1;

template <int NT>
__device__ __forceinline__ void group_plan(const DecodeParams& p, int* s) {
  static_assert(NT >= kBuckets / 2, "one scan wave covers the buckets");
  const int B = p.num_seqs;
  if (B > kRankMaxSeqs) return;
  const int32_t* lens = p.context_lens;
  int* base = s;
  int* cur = s + kPlanCur;
  int* key = s + kPlanPre;
  int* perm = s + kPlanPerm;
  for (int i = threadIdx.x; i < kBuckets; i += NT) cur[i] = 0;
  __syncthreads();
  for (int t = threadIdx.x; t < B; t += NT) atomicAdd(&cur[length_bucket(lens[t])], 1);
  __syncthreads();
  if (threadIdx.x < 64) {                                        // bucket bases, 2 buckets a lane
    const int l = threadIdx.x;
    const int c0 = cur[2 * l], c1 = cur[2 * l + 1];
    int inc = c0 + c1;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(inc, o);
      if (l >= o) inc += y;
    }
    const int exc = inc - c0 - c1;
    base[2 * l] = exc;
    base[2 * l + 1] = exc + c0;
    cur[2 * l] = exc;
    cur[2 * l + 1] = exc + c0;
  }
  __syncthreads();
  for (int t = threadIdx.x; t < B; t += NT) {                    // gather bucket members
    const int L = lens[t];
    key[atomicAdd(&cur[length_bucket(L)], 1)] = rank_key(L, t);
  }
  __syncthreads();
  for (int t = threadIdx.x; t < B; t += NT) {                    // rank inside the bucket
    const int L = lens[t];
    const int k = length_bucket(L), kk = rank_key(L, t);
    const int lo = base[k], hi = cur[k];
    int rank = lo;
    for (int j = lo; j < hi; ++j) rank += key[j] > kk;
    perm[rank] = t;
  }
  __syncthreads();
  for (int r = threadIdx.x; r < B; r += NT) key[r] = parts_of(p, lens[perm[r]]);
  __syncthreads();
  if (threadIdx.x < 64) wave_exclusive_scan(key, B);
  __syncthreads();
}

// Next item of this workgroup: false when the counter has passed the last one.
template <int NT>
__device__ __forceinline__ bool group_work(const DecodeParams& p, int* s, int& g, int& b, int& part,
                                           int& np) {
  if (threadIdx.x == 0) s[kPlanTicket] = atomicAdd(p.ws_ctr, 1);
  __syncthreads();
  const int ticket = __builtin_amdgcn_readfirstlane(s[kPlanTicket]);
  g = ticket % p.num_kv_heads;
  const int item = ticket / p.num_kv_heads;
  const int B = p.num_seqs;
  if (B > kRankMaxSeqs) {
    b = item / p.max_parts;
    part = item % p.max_parts;
    if (b >= B) return false;
    np = parts_of(p, p.context_lens[b]);
    return true;
  }
  const int* pre = s + kPlanPre;
  if (item >= __builtin_amdgcn_readfirstlane(pre[B])) return false;
  int lo = 0, hi = B - 1;                   // last rank whose first item is <= item
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (__builtin_amdgcn_readfirstlane(pre[mid]) <= item) lo = mid; else hi = mid - 1;
  }
  const int first = __builtin_amdgcn_readfirstlane(pre[lo]);
  b = __builtin_amdgcn_readfirstlane(s[kPlanPerm + lo]);
  part = item - first;
  np = __builtin_amdgcn_readfirstlane(pre[lo + 1]) - first;
  return true;
}

// A lane's cache slice of one token row: 16 bytes of a 16-bit or fp32 cache,
// or the 8 bytes of an FP8 cache that hold the same EPL elements.
template <DT kt> struct KvRaw { using type = u32x4; };
template <> struct KvRaw<DT::FP8> { using type = u32x2; };

template <DT dt, DT kt, int D, int G, int W, int MODE, int NB>
__global__ __launch_bounds__(64 * W)
void decode_kernel(DecodeParams p) {
  constexpr bool SPLIT = MODE != kSingle;
  constexpr bool GROUP = MODE == kGroupItems || MODE == kSpanItems;   // workgroup items, LDS merge
  constexpr bool SPAN = MODE == kSpanItems;
  constexpr bool F8 = kt == DT::FP8;        // e4m3 cache, widened to dt on the fly
  static_assert(F8 || kt == dt, "a 16-bit or fp32 cache has the query's type");
  static_assert(!F8 || dt != DT::F32, "an fp8 cache is read with 16-bit queries");
  using KR = typename KvRaw<kt>::type;
  constexpr int E = Elem<dt>::bytes;
  constexpr int KE = Elem<kt>::bytes;       // cache bytes per element
  constexpr int EPL = 16 / E;               // elements per lane per load
  constexpr int KB = EPL * KE;              // cache bytes per lane per load
  constexpr int LPR = D / EPL;              // lanes per token row
  constexpr int ROWS = 64 / LPR;            // rows per wave load
  constexpr int TPL = kBlockSize / ROWS;    // tokens per lane per block
  static_assert(LPR >= 8 && LPR <= 32 && TPL >= 1, "unsupported head_dim/dtype");
  static_assert(G <= LPR, "group larger than a row of lanes");
  using HM = HeadMap<G>;

  __shared__ __attribute__((aligned(16))) float s_acc[W][G][D];
  __shared__ float s_m[W][G];
  __shared__ float s_l[W][G];
  __shared__ int s_plan[GROUP ? kPlanInts : 1];

  const int lane = threadIdx.x & 63;
  // wave-uniform by construction; readfirstlane lets the compiler keep the
  // block walk (table reads, addresses, loop bounds) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane / LPR;
  const int c = lane % LPR;
  const int own = HM::owner(c);
  if constexpr (GROUP) group_plan<64 * W>(p, s_plan);
  // one trip, except with workgroup items: then one trip per item
  for (;;) {
  int g, b, part = 0, np = 1, Lb = 0;
  if constexpr (MODE == kWaveItems) {
    if (!split_work<64 * W>(p, wave, g, b, part)) return;   // no work item left
  } else if constexpr (GROUP) {
    if (!group_work<64 * W>(p, s_plan, g, b, part, np)) return;
  } else {
    g = blockIdx.x;
    b = sequence_of_row<64 * W>(p.context_lens, p.num_seqs, blockIdx.y, Lb);   // and its length
  }
  const int hq0 = g * G;

  // Fused decode step: the workgroup of (sequence b, kv head g) is the only one
  // that reads head g of b's newest row, so it writes that row itself (the
  // slot the table names for position L-1, as the append rule puts it) and a
  // barrier, whose workgroup-scope fences order the stores before every
  // wave's loads, separates the write from the attention.
  if constexpr (MODE == kSingle) {
    if (p.key_new) {                        // uniform: a kernel argument
      const int pos = Lb - 1;
      constexpr int NCH = D / 8;            // 8-element chunks of one head's row
      if (pos >= 0 && pos / kBlockSize < p.block_table_stride && threadIdx.x < 2 * NCH) {
        const int bid = p.block_tables[(int64_t)b * p.block_table_stride + pos / kBlockSize];
        if (bid >= 0 && bid < p.num_blocks) {
          const int kv = threadIdx.x / NCH, ch = threadIdx.x % NCH;
          const char* src = static_cast<const char*>(kv ? p.value_new : p.key_new) +
                            (int64_t)b * p.new_token_stride_bytes + ((int64_t)g * D + ch * 8) * E;
          char* dst = static_cast<char*>(const_cast<void*>(kv ? p.v_cache : p.k_cache)) +
                      (int64_t)bid * p.block_stride_bytes +
                      (((int64_t)(pos % kBlockSize) * p.num_kv_heads + g) * D + ch * 8) * KE;
          if constexpr (F8) {
            float x[8];
            unpack<dt>(load16(src), x);
            const float sc = (kv ? p.v_scale : p.k_scale)[g];
            uint32_t w[2] = {0u, 0u};
#pragma unroll
            for (int i = 0; i < 8; ++i) w[i >> 2] |= e4m3_encode(x[i] / sc) << (8 * (i & 3));
            *reinterpret_cast<u32x2*>(dst) = u32x2{w[0], w[1]};
          } else {
#pragma unroll
            for (int c16 = 0; c16 < E / 2; ++c16)   // 8 elements: one or two 16-byte chunks
              *reinterpret_cast<u32x4*>(dst + 16 * c16) = load16(src + 16 * c16);
          }
        }
      }
      __syncthreads();
    }
  }

  const int L = max(MODE == kSingle ? Lb : p.context_lens[b], 0);
  const int nblk = SPLIT ? split_blocks(p, L) : min((L + kBlockSize - 1) / kBlockSize, p.block_table_stride);
  // single pass and workgroup items: the W waves share the blocks round-robin.
  // wave items: every wave walks one partition on its own (no merge across waves)
  // span items: every wave walks one partition of the span on its own
  constexpr int STEP = MODE == kWaveItems || SPAN ? 1 : W;
  int lo = 0, hi = nblk;
  if constexpr (SPLIT) {
    lo = part * p.partition_blocks;
    if (lo >= nblk) {                       // only where empty pairs are numbered too
      if constexpr (GROUP) {
        __syncthreads();                    // every wave has read the ticket
        continue;
      } else {
        return;
      }
    }
    hi = min(nblk, lo + p.partition_blocks);
    if constexpr (SPAN) {                   // wave w: the w-th partition of the span (may be empty)
      const int sub = p.partition_blocks / W;
      lo = min(lo + wave * sub, hi);
      hi = min(hi, lo + sub);
    }
  }

  // this lane's 16-byte slice of the G query vectors, position i = head i ^ own
  u32x4 q[G];
  {
    const char* qb = static_cast<const char*>(p.query) +
                     (((int64_t)b * p.num_q_heads + hq0) * D + c * EPL) * E;
#pragma unroll
    for (int i = 0; i < G; ++i) q[i] = load16(qb + (int64_t)(i ^ own) * D * E);
  }
  // byte offsets of this lane's rows inside a physical block
  uint32_t off[TPL];
#pragma unroll
  for (int j = 0; j < TPL; ++j)
    off[j] = (uint32_t)((((r + ROWS * j) * p.num_kv_heads + g) * D) * KE + c * KB);

  // an fp8 cache stores K / k_scale and V / v_scale per kv head: k_scale folds
  // into the score scale and v_scale into the output
  const float sl2 = p.scale * kLog2e * (F8 ? p.k_scale[g] : 1.f);
  // constant address space: the uniform table lookups stay scalar loads even
  // where an asm statement below tells the compiler that memory may change
  const __attribute__((address_space(4))) int32_t* tbl =
      (const __attribute__((address_space(4))) int32_t*)(p.block_tables + (int64_t)b * p.block_table_stride);
  const char* kc = static_cast<const char*>(p.k_cache);
  const char* vc = static_cast<const char*>(p.v_cache);

  // softmax state of the owned head; accumulators by position
  float m_ref = -INFINITY, l = 0.f;
  float acc[G][EPL];
#pragma unroll
  for (int i = 0; i < G; ++i)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[i][e] = 0.f;

  // block id of logical block i (scalar load); ids are read two steps ahead of
  // their K/V loads so the dependent table lookup never stalls a block. Past
  // the end the last block is named again (the lookups and the loads of the
  // main loop are unconditional: a conditional load there would make the
  // compiler's wait counts drain the prefetch of every block); re-reading the
  // block a wave has just read is an L2 hit.
  // Walk order: where the waves of a workgroup share a range round-robin
  // (single pass, workgroup items) they start at a per-sequence offset into
  // it and wrap around, so sequences that share physical blocks do not all
  // read them at the same moment. Scores and masks follow the logical block,
  // so only the summation order changes.
  int rot = 0;
  if constexpr (MODE == kSingle || MODE == kGroupItems) {
    const int span = hi - lo;
    rot = span > 1 ? (int)(((uint32_t)b * 2654435761u) >> 8) % span : 0;
  }
  auto logical = [&](int i) -> int { return i + rot >= hi ? i + rot - (hi - lo) : i + rot; };
  auto block_id = [&](int i) -> int { return tbl[logical(min(i, hi - 1))]; };
  // K/V rows are read once per call: non-temporal loads keep them from
  // displacing reusable lines in L2 and the last-level cache (worth 5-8% on
  // the mixed-length fp16 batch)
  auto load_kv = [](const char* a) -> KR {
    return __builtin_nontemporal_load(reinterpret_cast<const KR*>(a));
  };
  auto fetch = [&](int bid, KR* kd, KR* vd) -> bool {
    const bool ok = (bid >= 0) && (bid < p.num_blocks);
    bid = ok ? bid : 0;                      // never address outside the pool
    const char* kb = kc + (int64_t)bid * p.block_stride_bytes;
    const char* vb = vc + (int64_t)bid * p.block_stride_bytes;
#pragma unroll
    for (int j = 0; j < TPL; ++j) kd[j] = load_kv(kb + off[j]);
#pragma unroll
    for (int j = 0; j < TPL; ++j) vd[j] = load_kv(vb + off[j]);
    return ok;
  };

  auto process = [&](int i, KR* kb, KR* vb, bool ok) {
    float x[TPL];
#pragma unroll
    for (int j = 0; j < TPL; ++j) {
      u32x4 kw;
      if constexpr (F8) kw = widen_fp8<dt>(kb[j]);
      else kw = kb[j];
      float v[G];
#pragma unroll
      for (int h = 0; h < G; ++h) v[h] = row_dot<dt>(q[h], kw);
      reduce_scatter<G, LPR>(v);
      x[j] = v[0] * sl2;
    }
    // Dead rows (past the end, or the whole block when its id is out of
    // range) may hold stale NaN: their scores become -inf and their V slices
    // never reach an accumulator. fp32 zeroes the slices; the 16-bit types
    // instead switch the byte selectors that split V into token pairs to the
    // constant-zero selector, which leaves the loaded registers untouched (no
    // copies, no early wait on the V loads).
    // An fp8 cache pairs bytes instead: [c j, c j+1, c+1 j, c+1 j+1] for
    // columns (4i, 4i+1) and (4i+2, 4i+3) of one dword, before widening.
    const int tok0 = logical(i) * kBlockSize;
    constexpr uint32_t kSelLo = F8 ? 0x05010400u : 0x05040100u;   // column 2i of tokens (j, j+1)
    constexpr uint32_t kSelHi = F8 ? 0x07030602u : 0x07060302u;   // column 2i+1
    constexpr uint32_t kKeepJ1 = F8 ? 0xFF00FF00u : 0xFFFF0000u;  // selector bytes of token j+1
    uint32_t sel_lo[TPL / 2 > 0 ? TPL / 2 : 1], sel_hi[TPL / 2 > 0 ? TPL / 2 : 1];
#pragma unroll
    for (int j = 0; j < TPL / 2; ++j) {
      sel_lo[j] = kSelLo;
      sel_hi[j] = kSelHi;
    }
    if (!ok || tok0 + kBlockSize > L) {      // uniform: only a sequence's last block
#pragma unroll
      for (int j = 0; j < TPL; ++j) {
        if (!ok || tok0 + r + ROWS * j >= L) {
          x[j] = -INFINITY;
          if constexpr (dt == DT::F32) {
            vb[j] = u32x4{0u, 0u, 0u, 0u};
          } else if ((j & 1) == 0) {         // byte selector 12 yields 0x00
            sel_lo[j / 2] = (sel_lo[j / 2] & kKeepJ1) | (0x0C0C0C0Cu & ~kKeepJ1);
            sel_hi[j / 2] = (sel_hi[j / 2] & kKeepJ1) | (0x0C0C0C0Cu & ~kKeepJ1);
          } else {
            sel_lo[j / 2] = (sel_lo[j / 2] & ~kKeepJ1) | (0x0C0C0C0Cu & kKeepJ1);
            sel_hi[j / 2] = (sel_hi[j / 2] & ~kKeepJ1) | (0x0C0C0C0Cu & kKeepJ1);
          }
        }
      }
    }

    bool need = false;
#pragma unroll
    for (int j = 0; j < TPL; ++j) need |= x[j] > m_ref + kRescaleSlack;
    if (__any(need)) {
      float mx = x[0];
#pragma unroll
      for (int j = 1; j < TPL; ++j) mx = fmaxf(mx, x[j]);
#pragma unroll
      for (int o = LPR; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
      const float mn = fmaxf(m_ref, mx);
      float cg[G];
      cg[0] = (m_ref == -INFINITY) ? 0.f : fast_exp2(m_ref - mn);
      l *= cg[0];
      m_ref = mn;
      all_gather<G>(cg);
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] *= cg[h];
    }

    const float mu = (m_ref == -INFINITY) ? 0.f : m_ref;
    if constexpr (dt == DT::F32) {
#pragma unroll
      for (int j = 0; j < TPL; ++j) {
        float pg[G];
        pg[0] = fast_exp2(x[j] - mu);
        l += pg[0];
        all_gather<G>(pg);
        float vf[EPL];
        unpack<dt>(vb[j], vf);
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(pg[h], vf[e], acc[h][e]);
      }
    } else {
      // 16-bit types: P·V on packed dot2 over the lane's token pairs (j, j+1).
      // The pair's probabilities are rounded to the input type once, in the
      // owning lane; the normaliser sums the same rounded values, so the
      // output stays a convex combination of the V rows.
#pragma unroll
      for (int j = 0; j < TPL; j += 2) {
        float pg[G];
        const uint32_t pk = pack2<dt>(fast_exp2(x[j] - mu), fast_exp2(x[j + 1] - mu));
        l = dot2_acc<dt>(pk, kOnes2<dt>, l);
        pg[0] = __uint_as_float(pk);
        all_gather<G>(pg);
        if constexpr (F8) {
#pragma unroll
          for (int i = 0; i < 2; ++i) {        // dword i: columns 4i .. 4i+3
            const uint32_t v0 = vb[j][i], v1 = vb[j + 1][i];
            const uint32_t lo = __builtin_amdgcn_perm(v1, v0, sel_lo[j / 2]);
            const uint32_t hi = __builtin_amdgcn_perm(v1, v0, sel_hi[j / 2]);
            const uint32_t col[4] = {widen_fp8_pair<dt, false>(lo), widen_fp8_pair<dt, true>(lo),
                                     widen_fp8_pair<dt, false>(hi), widen_fp8_pair<dt, true>(hi)};
#pragma unroll
            for (int h = 0; h < G; ++h) {
              const uint32_t ph = __float_as_uint(pg[h]);
#pragma unroll
              for (int k = 0; k < 4; ++k) acc[h][4 * i + k] = dot2_acc<dt>(ph, col[k], acc[h][4 * i + k]);
            }
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t v0 = vb[j][i], v1 = vb[j + 1][i];
            const uint32_t lo = __builtin_amdgcn_perm(v1, v0, sel_lo[j / 2]);   // column 2i of both tokens
            const uint32_t hi = __builtin_amdgcn_perm(v1, v0, sel_hi[j / 2]);   // column 2i+1
#pragma unroll
            for (int h = 0; h < G; ++h) {
              const uint32_t ph = __float_as_uint(pg[h]);
              acc[h][2 * i] = dot2_acc<dt>(ph, lo, acc[h][2 * i]);
              acc[h][2 * i + 1] = dot2_acc<dt>(ph, hi, acc[h][2 * i + 1]);
            }
          }
        }
      }
    }
  };

  // blocks first, first + STEP, ... through NB register buffers: all NB are in
  // flight before the first block is computed, and each buffer is refilled
  // with the block NB steps ahead as soon as it has been consumed. The loop
  // runs whole rounds of NB blocks and is left only at the end of a round, so
  // every path back to the loop head has issued the refills in the same order
  // as the prologue and the compiler's load counters wait only for the buffer
  // about to be used. Except with workgroup items, whose short round-robin
  // walks cannot spare the registers, the loop stops one round early so that
  // its refills all name blocks of the walk, and that last round refills only
  // the blocks that exist (its conditional loads come after the loop, where a
  // conservative wait costs nothing) instead of re-reading the last block.
  // The fewer than NB blocks left are computed last.
  constexpr bool EXACT_TAIL = MODE != kGroupItems;
  KR kbuf[NB][TPL], vbuf[NB][TPL];
  bool okb[NB];
  const int first = MODE == kWaveItems || SPAN ? lo : lo + wave;
  if (first < hi) {
    // buffers issued in order (an empty asm that clobbers memory keeps the
    // loads of buffer k+1 behind those of buffer k), as inside the loop
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      okb[k] = fetch(block_id(first + k * STEP), kbuf[k], vbuf[k]);
      asm volatile("" ::: "memory");
    }
    int bid = block_id(first + NB * STEP);
    int i = first;
    for (; i + ((EXACT_TAIL ? 2 : 1) * NB - 1) * STEP < hi; i += NB * STEP) {
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        process(i + k * STEP, kbuf[k], vbuf[k], okb[k]);
        // The refill must follow the last use of the buffer it overwrites:
        // were it hoisted, the register allocator would give the buffer two
        // homes, and the copies at the loop latch wait for every load in
        // flight. The accumulators pass through an empty asm that clobbers
        // memory, so the P.V that produces them completes before it and no
        // load moves above it.
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int e = 0; e < EPL; ++e) asm volatile("" : "+v"(acc[h][e])::"memory");
        okb[k] = fetch(bid, kbuf[k], vbuf[k]);
        bid = block_id(i + (k + NB + 1) * STEP);
      }
    }
    if constexpr (EXACT_TAIL) {
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        if (i + k * STEP < hi) {
          process(i + k * STEP, kbuf[k], vbuf[k], okb[k]);
          if (i + (k + NB) * STEP < hi) {
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
              for (int e = 0; e < EPL; ++e) asm volatile("" : "+v"(acc[h][e])::"memory");
            okb[k] = fetch(bid, kbuf[k], vbuf[k]);
            bid = block_id(i + (k + NB + 1) * STEP);
          }
        }
      }
      i += NB * STEP;
    }
#pragma unroll
    for (int k = 0; k + 1 < NB; ++k)
      if (i + k * STEP < hi) process(i + k * STEP, kbuf[k], vbuf[k], okb[k]);
  }

  // Sum the ROWS row-streams of the wave (lanes of one c share the head
  // order). l is summed in full. The accumulators are reduce-scattered: at the
  // exchange with lane ^ o (o = 32, 16, .., LPR) a lane keeps one half of the
  // values it still holds and hands the other half to its partner, so after
  // log2(ROWS) exchanges it owns NV = G*EPL/ROWS consecutive values (flattened
  // index head position * EPL + element) starting at vbase, which it stores
  // with wide writes; all 64 lanes store.
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1) l += __shfl_xor(l, o);
  constexpr int NV = G * EPL / ROWS;
  float vals[G * EPL];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) vals[h * EPL + e] = acc[h][e];
  int vbase = 0;
#pragma unroll
  for (int o = 32, n = G * EPL; o >= LPR; o >>= 1, n >>= 1) {
    const bool up = (lane & o) != 0;
#pragma unroll
    for (int i = 0; i < n / 2; ++i) {
      const float send = up ? vals[i] : vals[i + n / 2];
      const float keep = up ? vals[i + n / 2] : vals[i];
      vals[i] = keep + __shfl_xor(send, o);
    }
    vbase += up ? n / 2 : 0;
  }
  if constexpr (F8) {
    const float vs = p.v_scale[g];
#pragma unroll
    for (int i = 0; i < NV; ++i) vals[i] *= vs;
  }
  // the run of CW values at run index i: head position (vbase + i) / EPL,
  // elements from (vbase + i) % EPL (NV and EPL are multiples of CW)
  constexpr int CW = NV >= 4 ? 4 : NV;
  static_assert(NV % CW == 0 && EPL % CW == 0, "runs stay inside one head's row");
  auto store_run = [&](float* dst, int i) {
    if constexpr (CW == 4) *reinterpret_cast<f32x4*>(dst) = f32x4{vals[i], vals[i + 1], vals[i + 2], vals[i + 3]};
    else if constexpr (CW == 2) *reinterpret_cast<float2*>(dst) = float2{vals[i], vals[i + 1]};
    else *dst = vals[i];
  };
  if constexpr (MODE == kWaveItems) {       // the wave's partial goes straight to the workspace
    const int64_t row0 = (int64_t)b * p.num_q_heads + hq0;
#pragma unroll
    for (int i = 0; i < NV; i += CW) {
      const int v = vbase + i, hp = v / EPL, e = v % EPL;
      const int64_t pr = (row0 + (hp ^ own)) * p.max_parts + part;
      store_run(p.ws_acc + pr * D + c * EPL + e, i);
    }
    if (r == 0 && c < G) {                  // lanes 0..G-1 own distinct heads
      const int64_t pr = (row0 + own) * p.max_parts + part;
      p.ws_ml[2 * pr] = m_ref;
      p.ws_ml[2 * pr + 1] = l;
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < NV; i += CW) {
    const int v = vbase + i, hp = v / EPL, e = v % EPL;
    store_run(&s_acc[wave][hp ^ own][c * EPL + e], i);
  }
  if (r == 0 && c < G) {                    // lanes 0..G-1 own distinct heads
    s_m[wave][own] = m_ref;
    s_l[wave][own] = l;
  }
  __syncthreads();

  for (int idx = threadIdx.x; idx < G * D; idx += 64 * W) {
    const int h = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, s_m[w][h]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float mw = s_m[w][h];
      const float sc = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
      num = fmaf(sc, s_acc[w][h][d], num);
      den = fmaf(sc, s_l[w][h], den);
    }
    const int64_t row = (int64_t)b * p.num_q_heads + hq0 + h;
    if (GROUP && np > 1) {                  // a partition of a longer sequence: to the merge
      const int64_t pr = row * p.max_parts + part;
      p.ws_acc[pr * D + d] = num;
      if (d == 0) {
        p.ws_ml[2 * pr] = M;
        p.ws_ml[2 * pr + 1] = den;
      }
    } else {
      store_elem<dt>(p.out, row * D + d, den > 0.f ? num / den : 0.f);
    }
  }
  if constexpr (!GROUP) return;
  __syncthreads();                          // s_acc, s_m, s_l and the ticket are reused
  }
}

// Log-sum-exp merge of the split-KV partials: one workgroup of 256 threads per
// (query head, sequence). A thread owns 4 consecutive columns (one 16-byte
// load per partition) of every NPG-th partition, NPG = 256 / (D/4) partition
// groups run side by side, and the groups are combined through LDS:
//   M = max_p m_p,  w_p = 2^(m_p - M),  o = sum_p w_p acc_p / sum_p w_p l_p.
constexpr int kMergeThreads = 256;

template <DT dt, int D, bool DIRECT1>
__global__ __launch_bounds__(kMergeThreads)
void splitkv_merge_kernel(DecodeParams p) {
  constexpr int TPR = D / 4;                       // threads per partition row
  constexpr int NPG = kMergeThreads / TPR;         // partition groups
  __shared__ float s_max[kMergeThreads / 64];
  __shared__ float s_num[NPG][D];
  __shared__ float s_den[NPG];
  const int hq = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const int col = (t % TPR) * 4, grp = t / TPR;
  const int np = parts_of(p, p.context_lens[b]);
  if (DIRECT1 && np == 1) return;                  // written by the partition pass itself
  const int64_t row = (int64_t)b * p.num_q_heads + hq;
  const float* ml = p.ws_ml + row * p.max_parts * 2;
  const float* pa_ = p.ws_acc + row * p.max_parts * D;

  float M = -INFINITY;
  for (int i = t; i < np; i += kMergeThreads) M = fmaxf(M, ml[2 * i]);
  M = wave_max(M);
  if ((t & 63) == 0) s_max[t >> 6] = M;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kMergeThreads / 64; ++w) M = fmaxf(M, s_max[w]);

  f32x4 num = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
#pragma unroll 4
  for (int i = grp; i < np; i += NPG) {
    const float mi = ml[2 * i], li = ml[2 * i + 1];
    const float w = (mi == -INFINITY) ? 0.f : fast_exp2(mi - M);
    const f32x4 a = *reinterpret_cast<const f32x4*>(pa_ + (int64_t)i * D + col);
    den = fmaf(w, li, den);
#pragma unroll
    for (int k = 0; k < 4; ++k) num[k] = fmaf(w, a[k], num[k]);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) s_num[grp][col + k] = num[k];
  if (t % TPR == 0) s_den[grp] = den;
  __syncthreads();
  for (int d = t; d < D; d += kMergeThreads) {
    float n = 0.f, dn = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < NPG; ++g2) { n += s_num[g2][d]; dn += s_den[g2]; }
    store_elem<dt>(p.out, row * D + d, dn > 0.f ? n / dn : 0.f);
  }
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------
// Register buffers of K/V blocks in flight per wave. Two for every cache type:
// an fp8 buffer holds half the bytes, but four of them cost the grouped-query
// kernels a wave per SIMD (four heads a group: 144 against 118 VGPRs; eight:
// 196 against 164), which the GQA batch over an fp8 cache paid with 5% (102
// against 97 us); three buffers for a 16-bit cache were 4-6% slower on the
// same batch for the same reason.
constexpr int kDecodeBuffers = 2;

// Waves per workgroup.
constexpr int kDecodeWaves = 4;

// Split-KV takes workgroup items when no sequence has more than this many
// partitions (short or mixed contexts). Beyond it nearly every item is a whole
// partition: a 16-bit cache takes span items (W partitions per workgroup,
// merged in LDS, so a quarter of the partial rows reach the workspace), an
// fp8 cache wave items (its waves spend longer per block, and the barrier
// of the LDS merge costs more than the stores it saves).
constexpr int kGroupMaxParts = 16;

// Persistent grid of the workgroup-item kernel: as many workgroups as the chip
// holds at once, never more than there can be items.
template <typename K>
static int64_t resident_grid(K kernel, int threads, int64_t items) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess)
    return -1;
  return std::min<int64_t>(items, (int64_t)std::max(cus, 1) * std::max(per_cu, 1));
}

template <DT dt, DT kt, int D, int G, int MODE>
static hipError_t launch_mode(const DecodeParams& p_in, hipStream_t s) {
  constexpr int W = kDecodeWaves;
  auto kernel = decode_kernel<dt, kt, D, G, W, MODE, kDecodeBuffers>;
  // span items: the kernel and the merge see spans of W partitions as their
  // unit (the workspace keeps its stride of max_parts partition slots)
  DecodeParams p = p_in;
  p.max_blocks = p_in.max_parts * p_in.partition_blocks;
  if constexpr (MODE == kSpanItems) p.partition_blocks = W * p_in.partition_blocks;
  dim3 grid(p.num_kv_heads, p.num_seqs, 1);
  if constexpr (MODE != kSingle) {          // work items are handed out by a counter
    const int64_t items = (int64_t)p.num_kv_heads * p.num_seqs * p.max_parts;
    if (items + items / 4 + 64 * W > 0x7FFFFFFF) return hipErrorInvalidValue;   // tickets fit int32
    hipLaunchKernelGGL(splitkv_reset_kernel, dim3(1), dim3(64), 0, s, p.ws_ctr);
    int64_t wgs;
    if constexpr (MODE == kGroupItems || MODE == kSpanItems) {
      wgs = resident_grid(kernel, 64 * W, items);
      if (wgs < 0) return hipErrorInvalidValue;
    } else {
      wgs = (items + items / 4 + W - 1) / W;
    }
    grid = dim3((unsigned)std::max<int64_t>(wgs, 1));
  }
  hipLaunchKernelGGL(kernel, grid, dim3(64 * W), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || MODE == kSingle) return e;
  hipLaunchKernelGGL((splitkv_merge_kernel<dt, D, MODE != kWaveItems>), dim3(p.num_q_heads, p.num_seqs),
                     dim3(kMergeThreads), 0, s, p);
  return hipGetLastError();
}

template <DT dt, DT kt, int D, int MODE>
static hipError_t launch_g(const DecodeParams& p, hipStream_t s) {
  switch (p.num_q_heads / p.num_kv_heads) {
    case 1: return launch_mode<dt, kt, D, 1, MODE>(p, s);
    case 2: return launch_mode<dt, kt, D, 2, MODE>(p, s);
    case 4: return launch_mode<dt, kt, D, 4, MODE>(p, s);
    case 8: return launch_mode<dt, kt, D, 8, MODE>(p, s);
    default: return hipErrorInvalidValue;
  }
}

template <int MODE>
static hipError_t launch_any(const DecodeParams& p, hipStream_t s) {
  const DT dt = static_cast<DT>(p.dtype);
  if (static_cast<DT>(p.kv_dtype) == DT::FP8) {
    if (p.head_dim == 128) {
      if (dt == DT::F16) return launch_g<DT::F16, DT::FP8, 128, MODE>(p, s);
      if (dt == DT::BF16) return launch_g<DT::BF16, DT::FP8, 128, MODE>(p, s);
    } else if (p.head_dim == 64) {
      if (dt == DT::F16) return launch_g<DT::F16, DT::FP8, 64, MODE>(p, s);
      if (dt == DT::BF16) return launch_g<DT::BF16, DT::FP8, 64, MODE>(p, s);
    }
    return hipErrorInvalidValue;
  }
  if (p.kv_dtype != p.dtype) return hipErrorInvalidValue;
  if (p.head_dim == 128) {
    if (dt == DT::F32) return launch_g<DT::F32, DT::F32, 128, MODE>(p, s);
    if (dt == DT::F16) return launch_g<DT::F16, DT::F16, 128, MODE>(p, s);
    if (dt == DT::BF16) return launch_g<DT::BF16, DT::BF16, 128, MODE>(p, s);
  } else if (p.head_dim == 64) {
    if (dt == DT::F32) return launch_g<DT::F32, DT::F32, 64, MODE>(p, s);
    if (dt == DT::F16) return launch_g<DT::F16, DT::F16, 64, MODE>(p, s);
    if (dt == DT::BF16) return launch_g<DT::BF16, DT::BF16, 64, MODE>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t s) { return launch_any<kSingle>(p, s); }
hipError_t launch_decode_splitkv(const DecodeParams& p, hipStream_t s) {
  if (p.max_parts <= kGroupMaxParts) return launch_any<kGroupItems>(p, s);
  return p.kv_dtype == kKvFp8 ? launch_any<kWaveItems>(p, s) : launch_any<kSpanItems>(p, s);
}

}  // namespace pa
