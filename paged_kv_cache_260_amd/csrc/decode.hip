// Paged decode attention for CDNA4 (gfx950).
//
// What is computed: for each sequence s and query head h, exact softmax
// attention of q[s, h] over the sequence's cached K/V rows, which live in
// fixed-size blocks of a shared pool and are reached through the sequence's
// block table (vLLM paper page, "PagedAttention" core idea and block-pool
// diagram). The softmax is streamed with a running max and running sum, which
// gives the same result as standard attention (vLLM notes page,
// "FlashAttention": tiling plus online softmax, exact). Query heads that share
// a KV head (GQA/MQA, ICML-tutorial notes page) are processed together so each
// K/V tile is read from HBM once per group. Long sequences are split along the
// sequence into partitions (FlashDecoding, same tutorial page, kernel-
// optimisation part) whose partial results are merged by the last partition
// to finish, or by a separate merge kernel when a table allows more than
// kFusedMergeParts partitions.
//
// Work decomposition: one workgroup (4 waves) per work item = (KV head x
// query-head chunk, sequence, partition), items handed out longest first
// (make_plan / locate_item). Inside a workgroup the partition's 16-token
// tiles go round-robin to the waves; each wave keeps its own running max /
// sum / accumulator and the four are merged through LDS at the end.
//
// Per 16-token tile, per wave:
//   1. K and V tiles (16 x head_dim each) arrive by fully coalesced 16-byte
//      non-temporal loads into registers, issued one tile ahead.
//   2. Both go to wave-private LDS tiles (XOR-swizzled 16-byte chunks, bank
//      conflict free for the writes and the operand reads); the registers
//      then take the next tile's loads.
//   3. Transposed scores S^T[token][head] = K * Q^T (heads padded to 16) come
//      out of v_mfma_f32_16x16x32_{bf16,f16} (16x16x4 for fp32): lane (kg, n)
//      receives tokens 4kg..4kg+3 of head row n.
//   4. Online softmax in base 2 (scale * log2 e folded into one multiply)
//      against a reference max that is raised only when a score passes it by
//      more than 8 (so every weight stays <= 2^8); only then is the row max
//      taken across the four lanes of a row and the sums rescaled.
//   5. 16-bit storage: O^T += V^T P^T on v_mfma_f32_16x16x16. The weights a
//      lane holds are exactly its P^T operand (as hi + lo halves in the
//      storage type), so they stay in registers; V^T is read from LDS with
//      ds_read_b64_tr_b16. fp32 storage accumulates P * V on the VALU.
#include "attn_common.h"
#include "fp8_encode.h"
#include "kernels.h"
#include "tickets.h"

#include <math.h>

#include <algorithm>
#include <climits>
#include <atomic>

namespace pkv {
namespace {

using namespace attn;

// Batches of up to kCompactSeqs sequences (entities) take the longest-first
// item order below, built per workgroup in LDS.
constexpr int kCompactSeqs = 256;
static_assert(kHostPlanSeqs == kCompactSeqs, "a host-built order covers the batches a compact plan does");
constexpr int kCompactChunks = kCompactSeqs / 64;
constexpr int kRemBuckets = 8;

// The plan in LDS (int offsets from Cfg::kPlanOff):
//   entry[e] (kCompactSeqs of them) = (incl << 8) | rank, where incl is the
//         inclusive prefix of the full-partition counts in sequence order
//         (entity e owns full items [incl[e - 1], incl[e]); entries past the
//         batch hold the total) and rank the position of the entity's last
//         partition in the remainder list (< B <= 256; never matched past the
//         batch). compact_plan keeps incl below 2^23.
//   cnt:  per (bucket b, chunk c) entity counts at b * 4 + c, then the chunks'
//         full-partition totals at 36 + c;
//   aux:  shared mode, the chunks' longest private parts;
//   chg:  shared mode, per entity one bit: its sequence's prefix length
//         differs from the previous sequence's (64 bits per chunk);
//   bad:  shared mode, per chunk: a group of the chunk breaks the description.
constexpr int kPlanEntry = 0;
constexpr int kPlanCnt = kCompactSeqs;
constexpr int kPlanAux = kPlanCnt + (kRemBuckets + 1) * kCompactChunks + kCompactChunks;
constexpr int kPlanChg = kPlanAux + kCompactChunks;
constexpr int kPlanBad = kPlanChg + 2 * kCompactChunks;
constexpr int kPlanTicket = kPlanBad + kCompactChunks;  // a late workgroup's ticket
constexpr int kPlanInts = kPlanTicket + 1;
static_assert(kDecodeWaves == kCompactChunks, "one wave per 64-entity chunk of the plan");
static_assert((kRemBuckets + 1) * kCompactChunks <= 64, "bucket counts fit one wave");
static_assert(kCompactSeqs <= 256, "remainder ranks take 8 bits of a plan entry");

// Batches that take the longest-first plan: at most kCompactSeqs entities,
// and few enough partitions in all that the packed prefixes fit (partitions
// are at least 16 tokens, so the batch has fewer than 2^23 of them).
__host__ __device__ __forceinline__ bool compact_plan(const DecodeArgs &a) {
  // both terms evaluated (no short circuit): a workgroup then loads the three
  // sizes in one round trip instead of two
  return (a.num_seqs <= kCompactSeqs) & ((int64_t)a.num_seqs * a.max_blocks * a.block_size < (int64_t(1) << 27));
}

template <typename T, int D, int GT> struct Cfg {
  static constexpr int kEpc = Elem<T>::kPerChunk;        // elements per 16-byte chunk
  static constexpr int kCh = D / kEpc;                   // chunks per token row
  static constexpr int kLoads = kTileTokens * kCh / 64;  // 16-byte loads per lane per tile
  static constexpr int kSteps = kCh / 4;                 // QK MFMA steps per tile
  static constexpr int kRows = 64 / kCh;                 // token rows in the VALU V layout
  static constexpr int kNW = kDecodeWaves;
  // P*V on MFMA for 16-bit storage (V read transposed from LDS); fp32 storage
  // keeps P*V on the VALU.
  static constexpr bool kPvMfma = sizeof(T) == 2;
  static constexpr int kDimBlocks = D / 16;              // 16-dim output blocks (MFMA path)
  // LDS carve-up (bytes). Each wave owns one region: during the tile loop it
  // holds the staged K tile and the V tile (MFMA path) or P (VALU path);
  // afterwards the wave's partial accumulator (GT rows of D fp32) for the
  // workgroup merge.
  static constexpr int kKstBytes = kTileTokens * kCh * 16;
  static constexpr int kVstBytes = kPvMfma ? kTileTokens * kCh * 16 : 0;
  static constexpr int kPstBytes = kPvMfma ? 0 : kTileTokens * GT * 4;
  static constexpr int kStageBytes = kKstBytes + kVstBytes + kPstBytes;
  // rows of a wave's partial accumulator are padded by 16 bytes, so the
  // 16-byte stores of eight consecutive rows fall in distinct bank groups
  static constexpr int kAccRow = D + 4;  // floats
  static constexpr int kWaveBytes = kStageBytes > GT * kAccRow * 4 ? kStageBytes : GT * kAccRow * 4;
  static constexpr int kKstOff = 0;                      // within a wave region
  static constexpr int kVstOff = kKstBytes;
  static constexpr int kPstOff = kKstBytes + kVstBytes;
  static constexpr int kMlOff = kNW * kWaveBytes;        // workgroup-wide
  static constexpr int kBadOff = kMlOff + kNW * GT * 8;
  static constexpr int kFlagOff = kBadOff + kNW * 4;
  // shared mode: per member of the item, [0, 16) last-arrival flags, [16, 32)
  // slot totals, [32, 48) own slot base
  static constexpr int kMemOff = kFlagOff + 4;
  // Q of the item (its GT head rows, swizzled like a K tile), shared by the
  // four waves as the MFMA B operand of S^T = K Q^T; rows GT..15 of the
  // operand are zero
  static constexpr int kQOff = (kMemOff + 48 * 4 + 15) / 16 * 16;
  static constexpr int kQChunks = GT * kCh;
  static constexpr int kQPer = (kQChunks + kNW * 64 - 1) / (kNW * 64);  // Q chunks per thread
  // append mode: the newest token's K and V rows (2 kCh chunks)
  static constexpr int kNewOff = kQOff + kQChunks * 16;
  // the item order of compact plans (make_plan), kPlanInts ints
  static constexpr int kPlanOff = (kNewOff + 2 * kCh * 16 + 15) / 16 * 16;
  static constexpr int kSmem = kPlanOff + kPlanInts * 4;
  static_assert(kCh % 4 == 0 && 64 % kCh == 0, "head_dim must give 8, 16 or 32 chunks");
  static_assert(!kPvMfma || kCh == 8 || kCh == 16, "MFMA P*V path: 8 or 16 chunks per row");
  static_assert(GT >= 1 && GT <= 16, "head tile");
};

// Longest-first item order for batches of up to kCompactSeqs sequences.
// A sequence of L tokens has n = ceil(L / P) partitions: n - 1 full ones and
// a last one of L - (n - 1) P tokens. Item j of a unit is, in this order:
//   1. the full partitions of all sequences (sequence-major), then
//   2. the last partitions, in kRemBuckets buckets of decreasing length
//      (sequence order within a bucket); zero-length and invalid sequences
//      come last (their one item writes the zero or NaN row).
// Every workgroup derives the order from the lengths by itself (make_plan:
// one wave per 64-sequence chunk, wave-wide scans and ballots, two barriers)
// into LDS, where locate_item finds an item with four reads and ballots.

// What a work item's rows are (decode_item).
constexpr int kModeDecode = 0;
constexpr int kModeChunk = 1;
constexpr int kModePrefix = 2;
constexpr int kModeSuffix = 3;
constexpr int kModeShared = 4;
constexpr int kModeAppend = 5;

// The first loads of a plain decode or append item: the sequence length, the
// partition's block-table entries (one per lane), this thread's query chunks
// and (append) the new K/V row chunks. None of the addresses depends on the
// length. The item loop issues them for the next item as soon as the current
// item's tile loop is done, so they are in flight while the workgroup merges
// and writes the current item instead of after it.
template <int QPER> struct ItemHead {
  int L;
  int btv_raw;
  u32x4_t qv[QPER];
  u32x4_t new_chunk;
  bool ready;  // uniform: the fields hold the loads of the item about to run
};

struct ItemPlan {
  int full_items;  // full partitions of the batch (uniform)
  int items;       // all items of one unit (uniform)
  int p_pre;       // shared mode: partition length of the prefix entities (uniform)
  bool bad_desc;   // shared mode: the sharing description breaks its precondition (uniform)
};

// Shared mode: a prefix item's rows are at most this many (member, head)
// pairs, so a group has at most kSharedRows / group members.
constexpr int kSharedRows = 16;


// Inclusive prefix sum over the wave with DPP (no LDS round trips): shifts
// right by 1, 2, 4 and 8 within each 16-lane row (lanes shifted in from
// outside the row read 0), then row 0's total added to row 1 and row 2's to
// row 3 (row_bcast:15), then rows 0-1's total to rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1 and 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2 and 3
  return x;
}

// The length that orders an item is the number of tokens it walks: the
// sequence length (decode, chunk), the group's prefix length (prefix mode) or
// the tokens after the prefix (suffix mode).
// Shared mode: prefix partitions are cut about as long as the longest private
// part (rounded up to whole blocks), never shorter than the host's minimum
// (which keeps every row's slots within the in-kernel merge) and never longer
// than kMaxPartitionBlocks blocks. Items then take similar times, and a long
// prefix is not cut into more items than the private parts already give.
__device__ __forceinline__ int shared_prefix_partition(const DecodeArgs &a, int max_private) {
  if (a.prefix_partition_fixed) return a.prefix_partition_tokens;
  const int bs = a.block_size;
  int p = (max_private + bs - 1) / bs * bs;
  p = max(p, a.prefix_partition_tokens);
  return min(p, kMaxPartitionBlocks * bs);
}

// Builds the plan in LDS with the whole workgroup: wave c takes entities
// [64 c, 64 c + 64) (one load round trip), counts them per bucket, and after
// one barrier every wave turns the chunk counts into positions; a second
// barrier publishes them. Every workgroup computes the same plan.
template <int MODE>
__device__ __forceinline__ void make_plan(const DecodeArgs &a, ItemPlan &pl, int *sp, bool claim, uint32_t ticket) {
  const int lane = threadIdx.x & 63;
  const int c = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // this wave's chunk
  const int e = c * 64 + lane;                                            // this lane's entity
  const int B = a.num_seqs;
  const bool in = e < B;
  const int ec = min(e, B - 1);
  const int P = a.partition_tokens;
  const int64_t max_tok = (int64_t)a.max_blocks * a.block_size;
  int L;       // tokens the entity's items walk
  int Pe = P;  // its partition length
  pl.p_pre = a.prefix_partition_tokens;
  pl.bad_desc = false;
  if constexpr (MODE == kModeShared) {
    // entities: the groups' prefixes, then the sequences' private tokens
    const int ng = a.num_groups;
    const bool is_pre = e < ng;
    const int first = ec < ng ? a.query_start_loc[ec] : ec - ng;
    const int gend = ec < ng ? a.query_start_loc[ec + 1] : first + 1;
    const int m = min(max(first, 0), a.member_seqs - 1);
    const int len = a.seq_lens[m];
    const int pre = a.prefix_lens[m];
    // a private lane also reads the previous sequence's prefix length (its
    // own index is known, so this load goes out with the first ones)
    const int pre_prev = !is_pre && m > 0 ? a.prefix_lens[m - 1] : pre;
    // The arrival counts of the prefix and private partitions of a sequence
    // agree only if the description holds: the groups cut [0, member_seqs)
    // into consecutive ranges of at most kSharedRows / group members, and a
    // group's members share one prefix length. Each group lane checks its own
    // range here, and after the first barrier that no private lane inside it
    // saw the prefix length change from the sequence before; one violation
    // anywhere makes the whole call write NaN rows and count no arrivals, so
    // the counters stay at zero.
    bool bad = false;
    if (in && is_pre) {
      const int nmem = gend - first;
      bad = first < 0 || nmem < 1 || gend > a.member_seqs || nmem * a.group > kSharedRows ||
            (e == 0 && first != 0) || (e == ng - 1 && gend != a.member_seqs);
    }
    const unsigned long long chg = __builtin_amdgcn_ballot_w64(in && !is_pre && pre_prev != pre);
    L = is_pre ? pre : (pre >= 0 && pre <= len ? len - pre : -1);
    int max_private = !is_pre && in && (int64_t)len <= max_tok ? max(L, 0) : 0;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) max_private = max(max_private, __shfl_xor(max_private, d, 64));
    if (lane == 0) {
      sp[kPlanAux + c] = max_private;
      sp[kPlanChg + 2 * c] = (int)(uint32_t)chg;
      sp[kPlanChg + 2 * c + 1] = (int)(uint32_t)(chg >> 32);
    }
    __syncthreads();
#pragma unroll
    for (int cc = 0; cc < kCompactChunks; ++cc) max_private = max(max_private, sp[kPlanAux + cc]);
    if (in && is_pre && !bad) {
      // change bits of entities ng + first + 1 .. ng + gend - 1 (at most 15,
      // within two consecutive words of the bit array)
      const int b0 = ng + first + 1, b1 = ng + gend;  // [b0, b1), b1 <= kCompactSeqs
      if (b1 > b0) {
        const int wi = b0 >> 5;
        const uint64_t lo = (uint32_t)sp[kPlanChg + wi];
        const uint64_t hi = wi + 1 < 2 * kCompactChunks ? (uint32_t)sp[kPlanChg + wi + 1] : 0u;
        const uint64_t w = lo | (hi << 32);
        const uint64_t mask = ((1ull << (b1 - b0)) - 1ull) << (b0 & 31);  // b1 - b0 <= 15
        bad = (w & mask) != 0ull;
      }
    }
    const bool wave_bad = __builtin_amdgcn_ballot_w64(bad) != 0ull;  // every lane votes (outside the branch)
    if (lane == 0) sp[kPlanBad + c] = wave_bad ? 1 : 0;
    pl.p_pre = __builtin_amdgcn_readfirstlane(shared_prefix_partition(a, max_private));
    Pe = is_pre ? pl.p_pre : P;
  } else if constexpr (MODE == kModePrefix) {
    const int first = a.query_start_loc[ec];
    L = a.prefix_lens[min(max(first, 0), a.member_seqs - 1)];
  } else if constexpr (MODE == kModeSuffix) {
    const int len = a.seq_lens[ec];
    const int pre = a.prefix_lens[ec];
    L = pre >= 0 && pre <= len ? len - pre : -1;
  } else {
    L = a.seq_lens[ec];
  }
  const bool ok = in && L > 0 && (int64_t)L <= max_tok;
  const int full = ok ? (L - 1) / Pe : 0;
  const int rem = L - full * Pe;  // 1 .. Pe when ok
  // buckets of decreasing last-partition length; invalid and empty entities
  // in the last one, lanes past the batch in none (partitions are at most
  // 2^20 tokens, so the product fits 32 bits)
  const int bucket = !in ? 15 : (ok ? (Pe - rem) * kRemBuckets / Pe : kRemBuckets);
  const int x = wave_incl_scan(full);  // inclusive, within the chunk
  int pos_in = 0;                            // among the chunk's lanes of the same bucket
  int my_cnt = 0;                            // lane b: the chunk's lanes in bucket b
#pragma unroll
  for (int b = 0; b <= kRemBuckets; ++b) {
    const unsigned long long m = __builtin_amdgcn_ballot_w64(bucket == b);
    if (lane == b) my_cnt = __popcll(m);
    if (bucket == b)
      pos_in = __builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
  }
  if (lane <= kRemBuckets) sp[kPlanCnt + lane * kCompactChunks + c] = my_cnt;
  if (lane == 63) sp[kPlanCnt + (kRemBuckets + 1) * kCompactChunks + c] = x;
  // thread 0's ticket (its atomic returned with the lengths) for the workgroup
  if (claim && threadIdx.x == 0) sp[kPlanTicket] = (int)ticket;
  __syncthreads();
  // exclusive prefix over (bucket, chunk), bucket-major: the remainder list
  // takes bucket 0 of every chunk in chunk order, then bucket 1, ...
  const int v = lane < (kRemBuckets + 1) * kCompactChunks ? sp[kPlanCnt + lane] : 0;
  const int ex = wave_incl_scan(v) - v;
  int fbase = 0, ftot = 0;
#pragma unroll
  for (int cc = 0; cc < kCompactChunks; ++cc) {
    const int t = sp[kPlanCnt + (kRemBuckets + 1) * kCompactChunks + cc];
    fbase += cc < c ? t : 0;
    ftot += t;
  }
  const int rbase = __shfl(ex, min(bucket, kRemBuckets) * kCompactChunks + c, 64);
  sp[kPlanEntry + e] = ((in ? fbase + x : ftot) << 8) | (in ? rbase + pos_in : 0);
  __syncthreads();
  pl.full_items = __builtin_amdgcn_readfirstlane(ftot);
  pl.items = pl.full_items + B;
  if constexpr (MODE == kModeShared) {
#pragma unroll
    for (int cc = 0; cc < kCompactChunks; ++cc) pl.bad_desc |= sp[kPlanBad + cc] != 0;
  }
}

// Item j (< pl.items) of the order above -> (entity, partition), uniform:
// the first entity whose inclusive full count passes j (full list), or the
// entity of remainder rank j - full_items; four LDS reads and ballots.
__device__ __forceinline__ void locate_item(const ItemPlan &pl, const int *sp, int B, int j, int &s_out,
                                            int &p_out) {
  const int lane = threadIdx.x & 63;
  const bool full_list = j < pl.full_items;  // uniform
  const int jj = j - pl.full_items;
  int key[kCompactChunks];
#pragma unroll
  for (int c = 0; c < kCompactChunks; ++c) key[c] = sp[kPlanEntry + c * 64 + lane];
  int s_res = 0;
  bool found = false;
#pragma unroll
  for (int c = 0; c < kCompactChunks; ++c) {
    const bool hit = c * 64 + lane < B && (full_list ? (key[c] >> 8) > j : (key[c] & 255) == jj);
    const unsigned long long m = __builtin_amdgcn_ballot_w64(hit);
    if (!found && m != 0ull) {
      s_res = c * 64 + __builtin_ctzll(m);
      found = true;
    }
  }
  const int incl = sp[kPlanEntry + s_res] >> 8;
  const int excl = s_res > 0 ? sp[kPlanEntry + s_res - 1] >> 8 : 0;
  const int p = full_list ? j - excl : incl - excl;
  s_out = __builtin_amdgcn_readfirstlane(s_res);
  p_out = __builtin_amdgcn_readfirstlane(max(p, 0));
}

// Output value of a row from its own un-normalised state (M, num, den) and a
// second partial (pm = (m, l), pa = acc) of the same row:
//   (2^(M - M') num + 2^(m - M') pa) / (2^(M - M') den + 2^(m - M') l),
// M' = max(M, m); a state with max -inf contributes nothing; NaN propagates.
__device__ __forceinline__ float fold_partial(float M, float num, float den, float2 pm, float pa) {
  const float Mt = fmaxf(M, pm.x);
  const float f = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mt);
  const float fp = pm.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(pm.x - Mt);
  if (M != M || pm.x != pm.x) return __builtin_nanf("");
  return fmaf(f, num, fp * pa) / fmaf(f, den, fp * pm.y);
}

// One work item: query heads [hc GT, hc GT + GT) of KV head g (unit = g x
// head chunk hc) over tokens [part P, part P + P) of sequence s.
// F8: the pools hold OCP e4m3 codes with one scale per KV head (k_scale,
// v_scale); tiles are decoded to T on their way into LDS, k_scale is folded
// into the score scale and v_scale into the output (partials included).
// MODE selects what the item's rows are:
//   kModeDecode: query heads of sequence s, as above.
//   kModeChunk (GT = 16): the sequence's last n = qsl[s+1] - qsl[s] tokens are
//     queries, and the item's 16 rows are (chunk token, query head of g)
//     pairs, token-major from row 16 hc (unit = g x row block hc): row r is
//     token r / G, head g G + r % G. Chunk token i sits at position L - n + i
//     and sees tokens 0 .. L - n + i only, so each row carries its own last
//     visible token; the item's context ends after its last row's position.
//   kModePrefix (GT = 16): s is a group of sequences qsl[s] .. qsl[s+1] - 1
//     that share their first prefix_lens[qsl[s]] tokens (the same physical
//     blocks); rows are (member, query head of g) pairs laid out as in chunk
//     mode, all seeing the whole prefix, read once through the first member's
//     table. Results are un-normalised partials (pre_acc, pre_ml) per
//     (sequence, head) row, not outputs.
//   kModeSuffix: decode of sequence s over tokens [prefix_lens[s], L) only;
//     the row that finishes a (sequence, head) output folds in its prefix
//     partial (when prefix_lens[s] > 0).
//   kModeShared (GT = 16, one launch for both): entity s < num_groups is the
//     prefix of group s (as in kModePrefix, all members in one 16-row block,
//     partitions of prefix_partition_tokens); entity num_groups + i is the
//     private tokens of sequence i (rows: its G heads). Every partition of
//     either kind stores its rows' partial state in a slot of the (sequence,
//     head) row: prefix partition p in slot p, private partition p in slot
//     ceil(prefix / prefix partition) + p. The last partition to finish for a
//     (sequence, KV head) merges all of that row set's slots.
//   kModeAppend: decode as kModeDecode, and sequence s's newest token (position
//     L - 1) is appended first: its K and V rows come from k_new / v_new
//     [B, Hkv, D], are written to the slot the block table gives, and are used
//     from LDS (the copy in the pool is not read back).
// Issues the first loads of decode / append item (s, part) of `unit`
// (partitions of partition_tokens from token 0; Q rows past the head group
// are zero).
template <typename T, int D, int GT, int MODE>
__device__ __forceinline__ void load_item_head(const DecodeArgs &a, int tid, int unit, int s, int part,
                                               ItemHead<Cfg<T, D, GT>::kQPer> &h) {
  using C = Cfg<T, D, GT>;
  constexpr int kCh = C::kCh;
  const int lane = tid & 63;
  const int g = unit / a.head_chunks;
  const int hc = unit - g * a.head_chunks;
  const int nh = min(GT, a.group - hc * GT);
  const int jb = (part * a.partition_tokens) >> a.block_shift;
  const int32_t *bt_row = a.block_tables + (int64_t)s * a.max_blocks;
  h.btv_raw = jb + lane < a.max_blocks ? bt_row[jb + lane] : 0;
  const u32x4_t *qblk = reinterpret_cast<const u32x4_t *>(static_cast<const T *>(a.q) +
                                                          ((int64_t)s * a.n_heads + g * a.group + hc * GT) * D);
#pragma unroll
  for (int i = 0; i < C::kQPer; ++i) {
    const int u = tid + i * C::kNW * 64;
    h.qv[i] = u32x4_t{0u, 0u, 0u, 0u};
    if (u < C::kQChunks && u / kCh < nh) h.qv[i] = qblk[u];
  }
  // append mode: threads 0 .. 2 kCh - 1 fetch the new K (then V) row chunks
  // of (s, g), whatever partition this is (a few hundred bytes)
  h.new_chunk = u32x4_t{0u, 0u, 0u, 0u};
  if constexpr (MODE == kModeAppend) {
    if (tid < 2 * kCh) {
      const u32x4_t *src = static_cast<const u32x4_t *>(tid < kCh ? a.k_new : a.v_new);
      h.new_chunk = src[((int64_t)s * a.n_kv_heads + g) * kCh + (tid % kCh)];
    }
  }
  h.L = a.seq_lens[s];
  h.ready = true;
}

template <typename T, int D, int GT, bool F8, int MODE, bool HP = false>
__device__ __forceinline__ void decode_item(const DecodeArgs &a, char *smem, int tid, int unit, int s, int part,
                                            int p_pre, bool bad_desc, ItemHead<Cfg<T, D, GT>::kQPer> &hd,
                                            int s_next, int part_next) {
  using C = Cfg<T, D, GT>;
  // rows mode: item rows are (token or member, head) pairs
  constexpr bool RM = MODE == kModeChunk || MODE == kModePrefix || MODE == kModeShared;
  constexpr bool SH = MODE == kModeShared;
  // plain decode and append: the first loads come from (or go into) `hd`
  constexpr bool kHead = MODE == kModeDecode || MODE == kModeAppend;
  static_assert(!F8 || C::kPvMfma, "FP8 pools need a 16-bit query type");
  static_assert(!RM || (GT == 16 && C::kPvMfma), "chunk rows: 16-row tiles, 16-bit types");
  static_assert(MODE != kModeSuffix || C::kPvMfma, "shared-prefix decode: 16-bit types");
  static_assert(MODE != kModeAppend || C::kPvMfma, "append: 16-bit queries");
  constexpr int kKvBytes = F8 ? 1 : (int)sizeof(T);     // bytes per stored element
  constexpr int kL = kTileTokens * D * kKvBytes / (16 * 64);  // 16-byte loads per lane per K (or V) tile
  constexpr int kChKV = D * kKvBytes / 16;               // 16-byte chunks per stored token row
  constexpr int kCh = C::kCh;
  constexpr int kEpc = C::kEpc;
  constexpr int kNW = C::kNW;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int units = a.n_kv_heads * a.head_chunks;
  const int g = unit / a.head_chunks;
  const int hc = unit - g * a.head_chunks;
  const int H = a.n_heads;
  const int G = a.group;
  const int head0 = g * G + hc * GT;
  T *out = static_cast<T *>(a.out);
  // chunk rows: first query token of the sequence, chunk length, first row
  int q0 = 0, nq = 0;
  const int row0 = hc * GT;
  // rows mode with a bad range (a caller error): the item has no rows and
  // touches nothing
  bool bad_rows = false;
  // shared mode: a prefix entity (else the private tokens of sequence q0)
  const bool pre_item = SH && s < a.num_groups;
  if constexpr (SH) {
    if (pre_item) {
      q0 = a.query_start_loc[s];
      nq = a.query_start_loc[s + 1] - q0;
    } else {
      q0 = s - a.num_groups;
      nq = 1;
    }
    // a broken sharing description (make_plan): prefix items get no rows,
    // private items take the invalid-length path below (NaN rows, written by
    // each sequence's first private item); nothing counts an arrival. (Both
    // checks come after the item's first loads are issued: an early exit
    // here measured 1.6 us slower on the prompt-samples batch.)
    bad_rows = q0 < 0 || nq < 1 || q0 + nq > a.member_seqs || (pre_item && bad_desc);
  } else if constexpr (RM) {
    q0 = a.query_start_loc[s];
    nq = a.query_start_loc[s + 1] - q0;
    bad_rows = q0 < 0 || (MODE == kModePrefix && (nq < 1 || q0 + nq > a.member_seqs));
  }
  const int nh = RM ? (bad_rows ? 0 : max(0, min(GT, nq * G - row0))) : min(GT, G - hc * GT);
  // output (and query) row of item row i
  auto row_index = [&](int i) -> int64_t {
    if constexpr (RM) {
      const int r = row0 + i;
      return (int64_t)(q0 + r / G) * H + g * G + r % G;
    } else {
      return (int64_t)s * H + head0 + i;
    }
  };
  // partial-result row of item row i (split items)
  auto part_row = [&](int i) -> int64_t {
    if constexpr (SH) return row_index(i);
    else if constexpr (RM) return ((int64_t)s * units + unit) * GT + i;
    else return (int64_t)s * H + head0 + i;
  };
  float sl2 = a.scale_log2;  // scores in base-2 units
  float vsc = 1.f;           // output scale
  if constexpr (F8) {
    sl2 *= a.k_scale[g];
    vsc = a.v_scale[g];
  }

  const int P = pre_item ? p_pre : a.partition_tokens;
  // suffix mode (and private entities): the tokens start after the shared prefix
  int tok0 = 0;
  if constexpr (MODE == kModeSuffix) tok0 = a.prefix_lens[s];
  if constexpr (SH) tok0 = pre_item || bad_rows ? 0 : a.prefix_lens[q0];
  const int start = max(tok0, 0) + part * P;
  const int kg = lane >> 4;
  const int n = lane & 15;
  // Issue the length, the partition's table entries and q together; none of
  // these addresses depends on the length. Table entries past the sequence
  // (but inside the row) are read and ignored. Prefix mode reads the table
  // of the group's first member.
  const int jb = start >> a.block_shift;
  // Q chunks of this thread: chunk u = tid + 256 i of the GT x kCh head-row
  // block (rows past nh are zero)
  constexpr int kQPer = C::kQPer;
  u32x4_t qv[kQPer];
  int btv_raw;
  u32x4_t new_chunk = u32x4_t{0u, 0u, 0u, 0u};
  int L_head = 0;
  if constexpr (kHead) {
    if (!hd.ready) load_item_head<T, D, GT, MODE>(a, tid, unit, s, part, hd);
    btv_raw = hd.btv_raw;
#pragma unroll
    for (int i = 0; i < kQPer; ++i) qv[i] = hd.qv[i];
    new_chunk = hd.new_chunk;
    L_head = hd.L;
    hd.ready = false;
  } else {
  const int32_t *bt_row =
      a.block_tables + (int64_t)(MODE == kModePrefix || SH ? (bad_rows ? 0 : q0) : s) * a.max_blocks;
  btv_raw = jb + lane < a.max_blocks ? bt_row[jb + lane] : 0;
  if constexpr (RM) {
#pragma unroll
    for (int i = 0; i < kQPer; ++i) {
      const int u = tid + i * kNW * 64;
      qv[i] = u32x4_t{0u, 0u, 0u, 0u};
      if (u < C::kQChunks && u / kCh < nh)
        qv[i] = reinterpret_cast<const u32x4_t *>(static_cast<const T *>(a.q) + row_index(u / kCh) * D)[u % kCh];
    }
  } else {
    const u32x4_t *qblk = reinterpret_cast<const u32x4_t *>(static_cast<const T *>(a.q) +
                                                            ((int64_t)s * H + head0) * D);
#pragma unroll
    for (int i = 0; i < kQPer; ++i) {
      const int u = tid + i * kNW * 64;
      qv[i] = u32x4_t{0u, 0u, 0u, 0u};
      if (u < C::kQChunks && u / kCh < nh) qv[i] = qblk[u];
    }
  }
  }
  // no query rows: empty chunk, past its last row, or a bad range
  if (RM && nh == 0) return;
  // shared mode: members of the item (whole members only: G divides 16), and
  // for a prefix item each member's length and prefix (thread t < nmem)
  const int nmem = SH ? (pre_item ? nh / G : 1) : 0;
  int mem_len = 0, mem_pre = 0;
  if constexpr (SH) {
    if (pre_item && tid < nmem) {
      mem_len = a.seq_lens[q0 + tid];
      mem_pre = a.prefix_lens[q0 + tid];
    }
  }
  // Prefix mode: a prefix that is empty or not a whole number of blocks is
  // left to the suffix launch (nothing to fold, or NaN rows).
  const int L = kHead ? L_head
                      : (MODE == kModePrefix || pre_item ? a.prefix_lens[q0] : (SH ? a.seq_lens[q0] : a.seq_lens[s]));
  const int64_t cap = (int64_t)a.max_blocks * a.block_size;
  bool bad_len = L < 0 || (int64_t)L > cap;
  if constexpr (MODE == kModeChunk) bad_len |= L < nq || q0 < 0;
  if constexpr (HP) {
    // host-built order: the device length must give the partition count the
    // host planned for, or some partition has no item (or one too many): the
    // sequence then takes the invalid-length path in every item
    bad_len |= (!bad_len && L > 0 ? (L + P - 1) / P : 1) != (int)a.hp_np[s];
  }
  if constexpr (MODE == kModePrefix) bad_len |= (L & (a.block_size - 1)) != 0;
  if constexpr (MODE == kModeSuffix) bad_len |= tok0 < 0 || tok0 > L || (tok0 & (a.block_size - 1)) != 0;
  if constexpr (SH) {
    if (pre_item) bad_len |= (L & (a.block_size - 1)) != 0;
    else bad_len |= tok0 < 0 || tok0 > L || (tok0 & (a.block_size - 1)) != 0 || bad_desc;
  }
  if constexpr (MODE == kModePrefix) {
    if (bad_len || L == 0) return;
  } else if constexpr (SH) {
    // a prefix entity that is invalid or empty does nothing (its members'
    // private entities see the same prefix value: NaN rows, or no prefix);
    // a private entity that is invalid writes NaN rows; one with no private
    // token leaves its rows to the prefix partitions (zeros when empty)
    if (pre_item) {
      if (bad_len || L == 0) return;
    } else if (bad_len || L == tok0) {
      if (part == 0 && (bad_len || L == 0)) {
        const float v = bad_len ? __builtin_nanf("") : 0.f;
        for (int i = tid; i < nh * D; i += kNW * 64)
          out[row_index(i / D) * D + i % D] = static_cast<T>(v);
      }
      return;
    }
  } else if constexpr (MODE == kModeSuffix) {
    if (bad_len || L == tok0) {
      // invalid, or nothing after the prefix: the output is the prefix result
      // alone (zeros for an empty sequence)
      if (part == 0) {
        for (int i = tid; i < nh * D; i += kNW * 64) {
          const int64_t row = row_index(i / D);
          float v = bad_len ? __builtin_nanf("") : 0.f;
          if (!bad_len && tok0 > 0) {
            const float2 pm = a.pre_ml[row];
            v = a.pre_acc[row * D + i % D] / pm.y;
          }
          out[row * D + i % D] = static_cast<T>(v);
        }
      }
      return;
    }
  } else {
    if (bad_len || L == 0) {
      if (part == 0) {
        const float v = bad_len ? __builtin_nanf("") : 0.f;
        for (int i = tid; i < nh * D; i += kNW * 64)
          out[row_index(i / D) * D + i % D] = static_cast<T>(v);
      }
      return;
    }
  }
  // tokens the item's rows may see: [tok0, ctx)
  const int ctx = MODE == kModeChunk ? L - nq + (row0 + nh - 1) / G + 1 : L;
  // last visible token of this lane's row (lane % 16) (chunk rows)
  const int lim = (lane & 15) < nh ? L - nq + (row0 + (lane & 15)) / G : -1;
  if (start >= ctx) return;
  const int end = min(ctx, start + P);
  const int nparts = (ctx - tok0 + P - 1) / P;
  // append mode: this item holds the newest token when its partition is the
  // sequence's last
  const bool holds_new = MODE == kModeAppend && end == L;
  const int tok_new = L - 1;
  // shared mode: slot of this partition, and slot totals per member
  //   prefix partitions of a member: ceil(prefix / prefix partition)
  //   private partitions: ceil((L - prefix) / partition)
  const int npre_own = SH && !pre_item && tok0 > 0 ? (tok0 + p_pre - 1) / p_pre : 0;
  const int sbase = npre_own;  // prefix partitions come first
  int mem_tot = 0;             // thread t < nmem: slots of member t (0: not counted by this item)
  if constexpr (SH) {
    if (pre_item) {
      const bool ok = mem_pre == L && mem_len >= mem_pre && (int64_t)mem_len <= cap;
      mem_tot = ok ? nparts + (mem_len - mem_pre + a.partition_tokens - 1) / a.partition_tokens : 0;
    } else {
      mem_tot = npre_own + nparts;
    }
  }
  // Folds the prefix partial of output row `row` (dimension d) into this
  // row's own (M, num, den) and returns the output value (suffix mode).
  auto fold_prefix = [&](int64_t row, int d, float M, float num, float den) -> float {
    if (MODE != kModeSuffix || tok0 == 0) return num / den;
    return fold_partial(M, num, den, a.pre_ml[row], a.pre_acc[row * D + d]);
  };

  // Block ids of the partition (at most 64 table entries): lane i of btv holds
  // entry jb + i. They are read back with v_readlane, so the per-tile lookup
  // issues no memory operation and never waits on the K/V loads in flight.
  const int jmax = (end - 1) >> a.block_shift;  // last table entry this partition reads
  const int64_t kv_stride_blk = (int64_t)a.n_kv_heads * a.block_size;  // rows per physical block
  const int btv = jb + lane <= jmax ? btv_raw : 0;
  bool bad = false;

  auto tile_offset = [&](int ti) -> int64_t {  // offset of tile ti in 16-byte chunks (uniform)
    const int tok = ti * kTileTokens;
    const int j = (tok >> a.block_shift) - jb;
    int phys = __builtin_amdgcn_readlane(btv, j);
    if (phys < 0 || (int64_t)phys >= a.num_blocks) {
      bad = true;
      phys = 0;
    }
    return ((int64_t)phys * kv_stride_blk + (int64_t)g * a.block_size +
            (tok & (a.block_size - 1))) * kChKV;
  };
  const u32x4_t *kbase = static_cast<const u32x4_t *>(a.k_pool);
  const u32x4_t *vbase = static_cast<const u32x4_t *>(a.v_pool);
  struct Regs {
    u32x4_t k[kL];
    u32x4_t v[kL];
  };
  // K/V are read once per call: non-temporal loads keep them from displacing
  // other lines in L2 and the memory-side cache, which measures about 10%
  // faster for this gather than plain loads. `off` = tile_offset(tile).
  auto load_k = [&](int64_t off, Regs &r) {
#pragma unroll
    for (int i = 0; i < kL; ++i) r.k[i] = __builtin_nontemporal_load(kbase + off + i * 64 + lane);
  };
  auto load_v = [&](int64_t off, Regs &r) {
#pragma unroll
    for (int i = 0; i < kL; ++i) r.v[i] = __builtin_nontemporal_load(vbase + off + i * 64 + lane);
  };
  auto load_tile = [&](int ti, Regs &r) {
    const int64_t off = tile_offset(ti);
    load_k(off, r);
    load_v(off, r);
  };

  char *wreg = smem + wave * C::kWaveBytes;
  u32x4_t *kst = reinterpret_cast<u32x4_t *>(wreg + C::kKstOff);
  char *vst = wreg + C::kVstOff;
  char *pst = wreg + C::kPstOff;
  const u32x4_t *qs = reinterpret_cast<const u32x4_t *>(smem + C::kQOff);
  // slot of chunk ch of token tr in the staged K tile; FP8 staging writes a
  // lane's two chunks (2 c, 2 c + 1) in two passes, so its layout first moves
  // the chunk's low bit to the top: the eight lanes of a token then write
  // eight distinct bank groups in each pass
  auto kslot = [&](int tr, int ch) {
    if constexpr (F8) return kst_slot<kCh>(tr, (ch >> 1) | ((ch & 1) * (kCh / 2)));
    else return kst_slot<kCh>(tr, ch);
  };
  // 16-bit pools keep the wave's Q operand in registers for the whole item
  // (read from LDS once, after the workgroup has staged it) instead of
  // reading it from LDS for every tile
  constexpr bool kQReg = !F8 && C::kPvMfma;
  u32x4_t qreg[kQReg ? C::kSteps : 1];

  // Running softmax state of head row n, held by the four lanes (kg, n):
  // m is a reference max in base-2 units (the same in the four lanes), l this
  // lane's share (tokens 4 kg .. 4 kg + 3 of each tile) of the weight sum.
  float m = -INFINITY, l = 0.f;

  // Accumulators. MFMA path (O^T): acc[b][r] = O[head n][dim 16 b + 4 kg + r].
  // VALU path: accv[h][e] = partial O[head h][dim (lane % kCh) * kEpc + e] over
  // this lane's token row.
  f32x4_t acc[C::kPvMfma ? C::kDimBlocks : 1];
  float accv[C::kPvMfma ? 1 : GT][C::kPvMfma ? 1 : kEpc];
#pragma unroll
  for (int b = 0; b < (C::kPvMfma ? C::kDimBlocks : 1); ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int h = 0; h < (C::kPvMfma ? 1 : GT); ++h)
#pragma unroll
    for (int e = 0; e < (C::kPvMfma ? 1 : kEpc); ++e) accv[h][e] = 0.f;

  // MFMA path: this lane's byte offset for the transposed V reads. Source
  // lane (r = (lane % 16) / 4, q = lane % 4) of group kg addresses token
  // 4 kg + r, dims 16 b + 4q .. 4q + 3.
  const int tr_tok = 4 * kg + ((lane & 15) >> 2);
  const int tr_q = lane & 3;
  const int v_tr_base = tr_tok * kCh * 16 + tr_q * 8;
  const int v_tr_swz = vst_swz<kCh>(tr_tok);

  // The reference max may trail the true running max by up to kLazy (base-2
  // units), so every weight p = 2^(z - m) stays <= 2^kLazy. It is raised, and
  // the sums rescaled, only when a score passes it by more than that: the
  // result is unchanged (numerator and denominator share the reference) and
  // the common tile needs no cross-lane reduction.
  constexpr float kLazy = 8.f;

  // `has_next` (MFMA path): once the tile sits in LDS its registers are free,
  // so the loads of tile `next` go out into them before any math.
  // kEarlyK: the next K loads go out as soon as the K tile is staged, before
  // the V tile is. The tile loop then peels its last tile so that `has_next`
  // is a constant at each call: loads issued under a branch make the
  // compiler's wait counts assume the worst, and the V staging would wait
  // for the new K loads to land. Shared-prefix items, whose launch is short
  // and latency bound, gained 9% from it (39.6 -> 36.0 us on the
  // prompt-samples batch); the bandwidth-bound batches lost 1-2% (GQA 62.2 ->
  // 62.8 us, MHA 184.1 -> 188.0), and the peeled loop alone was within 1% either
  // way, so the other modes issue K and V together after both are staged.
  // (FP8 pools stay on the plain loop: the peeled one needs more than their
  // 128-register budget.)
  constexpr bool kEarlyK = MODE == kModeShared && !F8;
  auto process = [&](int ti, Regs &rg, int next, bool has_next) __attribute__((always_inline)) {
    const int valid = end - ti * kTileTokens;  // > 0; >= 16 means a full tile
    const bool partial = valid < kTileTokens;  // uniform
    // offset of the next tile, computed where its first load goes out
    const int64_t noff = C::kPvMfma && has_next && kEarlyK ? tile_offset(next) : 0;
    // stage K (coalesced order -> swizzled LDS tile); the MFMA path also stages
    // V, zeroing rows past the sequence (0 * NaN would poison the sum)
    if constexpr (F8) {
      // each 16-byte load holds 16 codes of one token: two chunks of T
      u32x4_t *vs = reinterpret_cast<u32x4_t *>(vst);
#pragma unroll
      for (int i = 0; i < kL; ++i) {
        const int u = i * 64 + lane;
        const int tr = u / kChKV;
        const int c8 = u - tr * kChKV;
        u32x4_t lo, hi;
        fp8x16_to<T>(rg.k[i], lo, hi);
        kst[kslot(tr, 2 * c8)] = lo;
        kst[kslot(tr, 2 * c8 + 1)] = hi;
      }
      if (has_next && kEarlyK) load_k(noff, rg);
#pragma unroll
      for (int i = 0; i < kL; ++i) {
        const int u = i * 64 + lane;
        const int tr = u / kChKV;
        const int c8 = u - tr * kChKV;
        u32x4_t lo, hi;
        // rows past the sequence: code 0 is +0 (four selects here instead of
        // eight on the decoded chunks)
        fp8x16_to<T>(partial && tr >= valid ? u32x4_t{0u, 0u, 0u, 0u} : rg.v[i], lo, hi);
        vs[tr * kCh + ((2 * c8) ^ vst_swz<kCh>(tr))] = lo;
        vs[tr * kCh + ((2 * c8 + 1) ^ vst_swz<kCh>(tr))] = hi;
      }
      if (has_next) {
        const int64_t off = kEarlyK ? noff : tile_offset(next);
        if (!kEarlyK) load_k(off, rg);
        load_v(off, rg);
      }
    } else {
#pragma unroll
    for (int i = 0; i < kL; ++i) {
      const int u = i * 64 + lane;
      kst[kst_slot<kCh>(u / kCh, u % kCh)] = rg.k[i];
    }
    if constexpr (C::kPvMfma) {
      if (has_next && kEarlyK) load_k(noff, rg);
      u32x4_t *vs = reinterpret_cast<u32x4_t *>(vst);
      if (!partial) {
#pragma unroll
        for (int i = 0; i < kL; ++i) {
          const int u = i * 64 + lane;
          vs[(u / kCh) * kCh + ((u % kCh) ^ vst_swz<kCh>(u / kCh))] = rg.v[i];
        }
      } else {
#pragma unroll
        for (int i = 0; i < kL; ++i) {
          const int u = i * 64 + lane;
          const int tr = u / kCh;
          vs[tr * kCh + ((u % kCh) ^ vst_swz<kCh>(tr))] =
              tr < valid ? rg.v[i] : u32x4_t{0u, 0u, 0u, 0u};
        }
      }
      if (has_next) {
        const int64_t off = kEarlyK ? noff : tile_offset(next);
        if (!kEarlyK) load_k(off, rg);
        load_v(off, rg);
      }
    }
    }
    if constexpr (MODE == kModeAppend) {
      // the newest token's rows replace what the tile load found in its slot
      if (holds_new && ti == tok_new / kTileTokens) {  // uniform
        const int tr = tok_new % kTileTokens;
        const u32x4_t *nr = reinterpret_cast<const u32x4_t *>(smem + C::kNewOff);
        if (lane < kCh) kst[kslot(tr, lane)] = nr[lane];
        else if (lane < 2 * kCh)
          reinterpret_cast<u32x4_t *>(vst)[tr * kCh + ((lane - kCh) ^ vst_swz<kCh>(tr))] = nr[lane];
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // S^T = K Q^T: lane (kg, n) receives tokens 4 kg + r of head row n, which
    // is also the layout P^T takes as the B operand of O^T += V^T P^T below,
    // so the weights never leave the registers
    f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < C::kSteps; ++c)
      sc = mfma_chunk<T>(kst[kslot(n, kg + 4 * c)],
                         kQReg ? qreg[kQReg ? c : 0] : (n < GT ? qs[kst_slot<kCh>(n, kg + 4 * c)] : u32x4_t{0u, 0u, 0u, 0u}),
                         sc);

    // scores in base-2 units; tokens past the sequence (chunk rows: past the
    // row's position) get -inf
    float z[4];
    bool over = false;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 4 * kg + r;
      if constexpr (MODE == kModeChunk)
        z[r] = t < valid && ti * kTileTokens + t <= lim ? sc[r] * sl2 : -INFINITY;
      else
        z[r] = t < valid ? sc[r] * sl2 : -INFINITY;
      over |= z[r] > m + kLazy;
    }
    if (__builtin_amdgcn_ballot_w64(over) != 0) {  // uniform: raise the reference
      // row max over the tile: this lane's four tokens, then the four lanes of the row
      const float mn = fmaxf(m, cols_max4(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]))));
      float alpha = __builtin_amdgcn_exp2f(m - mn);  // 0 on the first tile (m = -inf)
      // chunk rows may have seen nothing yet (mn = -inf): keep them empty
      if constexpr (MODE == kModeChunk) alpha = mn == -INFINITY ? 1.f : alpha;
      m = mn;
      l *= alpha;
      if constexpr (C::kPvMfma) {
#pragma unroll
        for (int b = 0; b < C::kDimBlocks; ++b) acc[b] *= alpha;
      } else {
#pragma unroll
        for (int h = 0; h < GT; ++h) {
          const float ah = readlane_f(alpha, h);
#pragma unroll
          for (int e = 0; e < kEpc; ++e) accv[h][e] *= ah;
        }
      }
    }
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = __builtin_amdgcn_exp2f(z[r] - m);
      if constexpr (MODE == kModeChunk) p[r] = z[r] == -INFINITY ? 0.f : p[r];  // also when m = -inf
      l += p[r];
    }

    if constexpr (C::kPvMfma) {
      // P^T as hi + lo in the storage type (about 16 mantissa bits together);
      // columns past the item's rows only feed output columns nobody reads
      typename Pv<T>::v4 hi, lo;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        hi[r] = static_cast<T>(p[r]);
        lo[r] = static_cast<T>(p[r] - static_cast<float>(hi[r]));
      }
#pragma unroll
      for (int b = 0; b < C::kDimBlocks; ++b) {
        const typename Pv<T>::v4 vb = lds_read_tr<T>(vst + v_tr_base + (((2 * b) ^ v_tr_swz) << 4));
        acc[b] = Pv<T>::mfma(vb, hi, acc[b]);
        acc[b] = Pv<T>::mfma(vb, lo, acc[b]);
      }
    } else {
      float *pstf = reinterpret_cast<float *>(pst);
      // p[token][head] -> LDS for the V layout
      if (n < GT) {
#pragma unroll
        for (int r = 0; r < 4; ++r) pstf[(4 * kg + r) * GT + n] = p[r];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int i = 0; i < kL; ++i) {
        const int tok = i * C::kRows + lane / kCh;
        float pv[GT];
#pragma unroll
        for (int h = 0; h < GT; ++h) pv[h] = pstf[tok * GT + h];
        float vf[kEpc];
        chunk_to_float<T>(rg.v[i], vf);
        if (partial && tok >= valid) {
#pragma unroll
          for (int e = 0; e < kEpc; ++e) vf[e] = 0.f;
        }
#pragma unroll
        for (int h = 0; h < GT; ++h)
#pragma unroll
          for (int e = 0; e < kEpc; ++e) accv[h][e] = fmaf(pv[h], vf[e], accv[h][e]);
      }
    }
  };

  // ---- stream this wave's tiles (tb + wave, tb + wave + NW, ...), one per
  // iteration. MFMA path: each iteration stages its tile in LDS, then issues
  // the next tile's loads into the same registers, so one tile is always in
  // flight and no load result crosses the loop edge unconsumed. VALU path:
  // load, then use.
  const int tb = start / kTileTokens;
  const int te = (end + kTileTokens - 1) / kTileTokens;
  Regs rg;
  if constexpr (C::kPvMfma) {
    if (tb + wave < te) load_tile(tb + wave, rg);
  }
  // the item's Q, shared by the waves, goes to LDS while those loads fly
#pragma unroll
  for (int i = 0; i < kQPer; ++i) {
    const int u = tid + i * kNW * 64;
    if (u < C::kQChunks)
      reinterpret_cast<u32x4_t *>(smem + C::kQOff)[kst_slot<kCh>(u / kCh, u % kCh)] = qv[i];
  }
  // append mode: the new rows go to LDS for the tile that holds the token;
  // the pool copy (head chunk 0 only, at the slot the table gives) is stored
  // after the tile loop, so no wait on it sits in front of the K/V loads
  int new_phys = -1;
  uint2 new_codes = make_uint2(0u, 0u);  // FP8 pools: this thread's 8 codes of the new row
  if constexpr (MODE == kModeAppend) {
    if (holds_new) {
      u32x4_t staged = new_chunk;
      if constexpr (F8) {
        // encode as the FP8 cache write does (x * (1 / scale), nearest e4m3),
        // and stage the codes decoded exactly, as a tile load of the written
        // slot would
        if (tid < 2 * kCh) {
          const float inv = __fdiv_rn(1.0f, (tid < kCh ? a.k_scale : a.v_scale)[g]);
          const T *e = reinterpret_cast<const T *>(&new_chunk);
          uint32_t w[2] = {0u, 0u};
#pragma unroll
          for (int j = 0; j < 8; ++j) w[j >> 2] |= f32_to_e4m3(__fmul_rn(static_cast<float>(e[j]), inv)) << (8 * (j & 3));
          new_codes = make_uint2(w[0], w[1]);
          uint32_t d[4];
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            d[2 * i] = fp8x2_to<T>(w[i], false);
            d[2 * i + 1] = fp8x2_to<T>(w[i], true);
          }
          staged = u32x4_t{d[0], d[1], d[2], d[3]};
        }
      }
      if (tid < 2 * kCh) reinterpret_cast<u32x4_t *>(smem + C::kNewOff)[tid] = staged;
      const int phys = __builtin_amdgcn_readlane(btv, (tok_new >> a.block_shift) - jb);
      if (hc == 0 && phys >= 0 && (int64_t)phys < a.num_blocks) new_phys = phys;
    }
  }
  int *mflag = reinterpret_cast<int *>(smem + C::kMemOff);  // shared mode: [16] flags
  int *mtot = mflag + 16;                                     // [16] slot totals per member
  if constexpr (SH) {
    if (tid < 16) mtot[tid] = tid < nmem ? mem_tot : 0;
  }
  __syncthreads();
  if constexpr (kQReg) {
#pragma unroll
    for (int c = 0; c < C::kSteps; ++c) qreg[c] = n < GT ? qs[kst_slot<kCh>(n, kg + 4 * c)] : u32x4_t{0u, 0u, 0u, 0u};
  }
  // streaming runs at normal priority; the latency chains around it (plan,
  // item start, merge) run raised, so a SIMD's streaming waves do not hold
  // them up
  __builtin_amdgcn_s_setprio(0);
  if constexpr (kEarlyK) {
    int ti = tb + wave;
    for (; ti + kNW < te; ti += kNW) process(ti, rg, ti + kNW, true);
    if (ti < te) process(ti, rg, -1, false);
  } else if constexpr (C::kPvMfma) {
    for (int ti = tb + wave; ti < te; ti += kNW) {
      const int next = ti + kNW < te ? ti + kNW : -1;
      process(ti, rg, next, next >= 0);
    }
  } else {
    for (int ti = tb + wave; ti < te; ti += kNW) {
      load_tile(ti, rg);
      process(ti, rg, -1, false);
    }
  }
  __builtin_amdgcn_s_setprio(2);

  // the next item's first loads fly while this one is merged and written
  if constexpr (kHead) {
    if (s_next >= 0) {
      load_item_head<T, D, GT, MODE>(a, tid, unit, s_next, part_next, hd);
    } else {
      hd = ItemHead<kQPer>{};
    }
  }
  if constexpr (MODE == kModeAppend) {
    if (new_phys >= 0 && tid < 2 * kCh) {
      const int64_t row = (int64_t)new_phys * kv_stride_blk + (int64_t)g * a.block_size + (tok_new & (a.block_size - 1));
      if constexpr (F8) {
        // D codes per row: this thread's 8 at byte (tid % kCh) * 8
        uint2 *dst = reinterpret_cast<uint2 *>(static_cast<uint8_t *>(const_cast<void *>(tid < kCh ? a.k_pool : a.v_pool)) +
                                               row * D) + (tid % kCh);
        *dst = new_codes;
      } else {
        u32x4_t *dst = static_cast<u32x4_t *>(const_cast<void *>(tid < kCh ? a.k_pool : a.v_pool));
        dst[row * kCh + (tid % kCh)] = reinterpret_cast<const u32x4_t *>(smem + C::kNewOff)[tid];
      }
    }
  }

  // ---- wave totals to LDS
  l = cols_sum4(l);
  // the wave's staging area is free now: it takes the wave's partial sums
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float *macc = reinterpret_cast<float *>(wreg);
  float2 *mml = reinterpret_cast<float2 *>(smem + C::kMlOff) + wave * GT;
  int *mbad = reinterpret_cast<int *>(smem + C::kBadOff);
  if constexpr (C::kPvMfma) {
    if (n < GT) {
#pragma unroll
      for (int b = 0; b < C::kDimBlocks; ++b)
        *reinterpret_cast<f32x4_t *>(macc + n * C::kAccRow + 16 * b + 4 * kg) = acc[b];
    }
  } else {
    // token-row sums of the VALU accumulators
#pragma unroll
    for (int h = 0; h < GT; ++h)
#pragma unroll
      for (int e = 0; e < kEpc; ++e)
#pragma unroll
        for (int off = kCh; off < 64; off <<= 1) accv[h][e] += __shfl_xor(accv[h][e], off, 64);
    if (lane < kCh) {
#pragma unroll
      for (int h = 0; h < GT; ++h)
#pragma unroll
        for (int e = 0; e < kEpc; ++e) macc[h * C::kAccRow + lane * kEpc + e] = accv[h][e];
    }
  }
  if (kg == 0 && n < GT) mml[n] = make_float2(m, l);
  if (lane == 0) mbad[wave] = bad ? 1 : 0;
  __syncthreads();

  // ---- merge the waves: thread t owns output elements t, t + 256, ... of the
  // nh x D block (head-major); kPer of them at most
  constexpr int kPer = (GT * D + kNW * 64 - 1) / (kNW * 64);
  auto acc_of = [&](int w) { return reinterpret_cast<const float *>(smem + w * C::kWaveBytes); };
  const float2 *ml_all = reinterpret_cast<const float2 *>(smem + C::kMlOff);
  int any_bad = 0;
#pragma unroll
  for (int w = 0; w < kNW; ++w) any_bad |= mbad[w];
  // shared mode: every split row is merged in the kernel (at most
  // kFusedMergeParts slots); skip the arrival step when no member is split
  bool any_split = false;
  if constexpr (SH) {
    for (int t = 0; t < nmem; ++t) any_split |= mtot[t] > 1;
  }
  const bool fused = SH ? any_split : (nparts > 1 && a.arrivals != nullptr);
  float rM[kPer], rnum[kPer], rden[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int idx = tid + k * kNW * 64;
    rM[k] = -INFINITY;
    rnum[k] = rden[k] = 0.f;
    if (idx >= nh * D) continue;
    const int h = idx / D;
    const int d = idx - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kNW; ++w) M = fmaxf(M, ml_all[w * GT + h].x);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < kNW; ++w) {
      const float2 ml = ml_all[w * GT + h];
      const float f = ml.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml.x - M);
      den = fmaf(f, ml.y, den);
      num = fmaf(f, acc_of(w)[h * C::kAccRow + d], num);
    }
    if constexpr (F8) num *= vsc;
    if (any_bad) {
      num = den = M = __builtin_nanf("");
    }
    rM[k] = M;
    rnum[k] = num;
    rden[k] = den;
    // slots of this row's (sequence, head) and this partition's own slot
    const int tot = SH ? mtot[h / G] : nparts;
    const int own = SH ? sbase + part : part;
    if (SH && tot == 0) continue;  // member not counted here (invalid)
    if (tot == 1) {
      if constexpr (MODE == kModePrefix) {
        const int64_t row = row_index(h);
        a.pre_acc[row * D + d] = num;
        if (d == 0) a.pre_ml[row] = make_float2(M, den);
      } else {
        out[row_index(h) * D + d] = static_cast<T>(fold_prefix(row_index(h), d, M, num, den));
      }
    } else {
      const int64_t pi = part_row(h) * a.max_parts + own;
      if (!fused) {
        a.part_acc[pi * D + d] = num;
        if (d == 0) a.part_ml[pi] = make_float2(M, den);
      } else {
        // agent-scope stores: written through to memory, where the last
        // partition of the sequence (possibly on another XCD) reads them
        __hip_atomic_store(a.part_acc + pi * D + d, num, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (d == 0)
          __hip_atomic_store(reinterpret_cast<unsigned long long *>(a.part_ml + pi),
                             __builtin_bit_cast(unsigned long long, make_float2(M, den)),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  if (!fused) return;

  // ---- split sequence, merged by the last of its partitions to finish.
  // Every partition's partial stores are complete (waited for) before the
  // workgroup's arrival is counted, so the partition whose increment returns
  // nparts - 1 finds all the other partials in memory; it reads them with
  // agent-scope loads (never stale lines of its XCD's L2), resets the counter
  // for the next call and writes the merged rows:
  //   M = max_p m_p,  out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p.
  //
  // Ordering. No fence is used; the argument rests on how gfx950 executes
  // these accesses, not on the language memory model (where relaxed atomics
  // alone would not order the partial stores before the increment):
  //   - agent-scope atomic stores and loads bypass the XCD-local L2 for
  //     coherence (stores write through, loads miss to memory), so a store
  //     that has completed is visible to an agent-scope load from any XCD;
  //   - a wave's vector-memory stores count in vmcnt until the memory side
  //     acknowledges them, so "s_waitcnt vmcnt(0)" below returns only after
  //     every partial store of this wave has completed, and the barrier after
  //     it extends that to the workgroup before thread 0 increments;
  //   - the last arriver's loads are issued only after its increment has
  //     returned (they depend on its value through the flag in LDS).
  // The release/acquire pair the compiler would emit adds a writeback and an
  // invalidate of the whole L2 around plain stores, which this data does not
  // need; it measured 3-10x slower.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  int *flag = reinterpret_cast<int *>(smem + C::kFlagOff);
  if constexpr (SH) {
    // one counter per (member sequence, KV head); each split member counts
    // this partition once
    int any_last = 0;
    if (tid < nmem) {
      const int t = mtot[tid];
      int last = 0;
      if (t > 1) {
        int32_t *cnt = a.arrivals + (int64_t)(q0 + tid) * a.n_kv_heads + g;
        const int prev = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = prev == t - 1;
        if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      mflag[tid] = last;
      any_last = last;
    }
    if (tid == 0) *flag = 0;
    __syncthreads();
    if (any_last) *flag = 1;  // benign race: every writer stores 1
    __syncthreads();
  } else if (tid == 0) {
    int32_t *cnt = a.arrivals + (int64_t)s * units + unit;
    const int prev = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = prev == nparts - 1;
    if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = last;
  }
  if constexpr (!SH) __syncthreads();
  if (!*flag) return;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int idx = tid + k * kNW * 64;
    if (idx >= nh * D) continue;
    const int h = idx / D;
    const int d = idx - h * D;
    const int64_t prow = part_row(h);
    if (SH && !mflag[h / G]) continue;  // this member is merged by another partition
    const int tot = SH ? mtot[h / G] : nparts;
    const int own = SH ? sbase + part : part;
    // the partials in slot order, this partition's own from registers: the
    // sums do not depend on which partition happened to finish last
    float2 oml[kFusedMergeParts];
    float ox[kFusedMergeParts];
#pragma unroll
    for (int p = 0; p < kFusedMergeParts; ++p) {
      oml[p] = make_float2(-INFINITY, 0.f);
      ox[p] = 0.f;
      if (p == own) {
        oml[p] = make_float2(rM[k], rden[k]);
        ox[p] = rnum[k];
      } else if (p < tot) {
        const int64_t pi = prow * a.max_parts + p;
        oml[p] = __builtin_bit_cast(
            float2, __hip_atomic_load(reinterpret_cast<unsigned long long *>(a.part_ml + pi),
                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        ox[p] = __hip_atomic_load(a.part_acc + pi * D + d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    float M = -INFINITY;
    bool bad = false;
#pragma unroll
    for (int p = 0; p < kFusedMergeParts; ++p) {
      bad |= oml[p].x != oml[p].x;
      M = fmaxf(M, oml[p].x);
    }
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int p = 0; p < kFusedMergeParts; ++p) {
      const float f = oml[p].x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(oml[p].x - M);
      den = fmaf(f, oml[p].y, den);
      num = fmaf(f, ox[p], num);
    }
    if constexpr (MODE == kModePrefix) {
      const int64_t row = row_index(h);
      a.pre_acc[row * D + d] = bad ? __builtin_nanf("") : num;
      if (d == 0) a.pre_ml[row] = make_float2(bad ? __builtin_nanf("") : M, den);
    } else {
      if (bad) M = num = den = __builtin_nanf("");
      out[row_index(h) * D + d] = static_cast<T>(fold_prefix(row_index(h), d, M, num, den));
    }
  }
}

// Three workgroups per CU (12 waves). Bandwidth alone would not need them
// (a gather of 4 KiB tiles reaches the chip's read rate with 2 workgroups of
// 4 waves per CU, one tile in flight per wave), but every item also has
// latency-bound phases (plan, first loads, merge), and more resident
// workgroups keep more items streaming while others are in those phases:
// 2 per CU measured 3% slower on the GQA batch-128 step, 1 per CU 28%. The
// register budget is pinned so the item loop does not trade occupancy for
// registers. fp32 storage with large head tiles needs more registers.
// Waves per SIMD the register budget is set for: 16-bit pools 3 (at 4 the
// tile loop no longer fits its registers and runs much slower), FP8 pools 4
// (half the bytes per tile, so more waves keep more bytes in flight; their
// LDS fits 4 workgroups per CU).
template <typename T, int D, int GT, bool F8> constexpr int decode_waves_per_eu() {
  return F8 ? 4 : (sizeof(T) == 2 || GT <= 4) ? 3 : 2;
}

template <typename T, int D, int GT, bool F8, int MODE, bool HP = false>
__global__ __launch_bounds__(kDecodeWaves * 64)
__attribute__((amdgpu_waves_per_eu(decode_waves_per_eu<T, D, GT, F8>()))) void paged_decode_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[Cfg<T, D, GT>::kSmem];
  // Work items. The hardware deals workgroup i to XCD i % 8, and workgroups
  // start in index order as slots free up. The unit (KV head x query-head
  // chunk) varies fastest, so the sequences a KV head serves stay on one XCD
  // and its L2 (shared-prefix blocks are read together). For batches of up to
  // kCompactSeqs sequences, the wgs_per_unit workgroups of a unit walk that
  // unit's items in longest-first order (make_plan), in boustrophedon rounds:
  // workgroup w takes items w, 2G - 1 - w, 2G + w, ... (G = wgs_per_unit), so
  // a workgroup that drew a long item early draws a short one next, and no
  // workgroup is launched for the partitions that short sequences do not have.
  // Larger batches take one item per workgroup in a fixed order:
  // partition-major, the sequence rotated by the partition so the partitions
  // of a long sequence spread over the chip.
  __builtin_amdgcn_s_setprio(2);
  const int units = a.n_kv_heads * a.head_chunks;
  const bool compact = HP || compact_plan(a);  // a host-built order implies a compact plan
  // A workgroup past the first static_wgs takes the place of workgroup
  // static_wgs + ticket_place(ticket): the claimers together cover exactly
  // those places, in the order their slots free up on any XCD, whatever value
  // the counter starts from (tickets.h; a clean call leaves it where it
  // started). The fixed map sends workgroup i to XCD i mod 8, and XCDs finish
  // their equal shares several microseconds apart; tickets let the later,
  // shorter items go to the XCDs that are ahead.
  const bool claim = compact && a.tickets != nullptr && (int64_t)blockIdx.x >= a.static_wgs;
  const uint32_t claimers = gridDim.x - (uint32_t)a.static_wgs;  // >= 1 whenever tickets are on
  uint32_t ticket = 0;
  if (claim && threadIdx.x == 0)
    ticket = __builtin_amdgcn_atomic_inc32(a.tickets, claimers - 1u, __ATOMIC_RELAXED, "agent");
  ItemPlan plan;
  plan.p_pre = a.prefix_partition_tokens;
  plan.full_items = plan.items = 0;
  plan.bad_desc = false;
  int *plan_lds = reinterpret_cast<int *>(smem + Cfg<T, D, GT>::kPlanOff);
  // HP: the work order comes built from the host (one item per workgroup)
  // and replaces the plan, so no workgroup waits on the lengths before its
  // first item's loads; claimers still share their ticket.
  if constexpr (HP) {
    plan.items = a.hp_items;
    if (claim) {
      if (threadIdx.x == 0) plan_lds[kPlanTicket] = (int)ticket;
      __syncthreads();
    }
  } else {
    if (compact) make_plan<MODE>(a, plan, plan_lds, claim, ticket);
  }
  // item j (< plan.items) -> (sequence, partition)
  auto locate = [&](int j, int &s_out, int &p_out) {
    if constexpr (HP) {
      const int e = a.hp[j];
      s_out = e & 255;
      p_out = e >> 8;
    } else {
      locate_item(plan, plan_lds, a.num_seqs, j, s_out, p_out);
    }
  };
  // Tickets place items only when every workgroup takes one item (a unit has
  // no more items than workgroups); with two or more rounds per workgroup the
  // fixed places measured faster. Every claimer has drawn its ticket either
  // way, so the counter still wraps to zero.
  const bool placed = claim && plan.items <= a.wgs_per_unit;
  const int64_t lin =
      placed ? (int64_t)a.static_wgs +
                   ticket_place((uint32_t)__builtin_amdgcn_readfirstlane(plan_lds[kPlanTicket]), claimers)
             : (int64_t)blockIdx.x;
  const int unit = (int)(lin % units);
  const int w = (int)(lin / units);
  ItemHead<Cfg<T, D, GT>::kQPer> hd{};
  hd.ready = false;
  // item j of this workgroup's walk (compact plans), or -1 past its end
  auto item_of = [&](int round) -> int64_t {
    const int G = a.wgs_per_unit;
    const int64_t j = (int64_t)round * G + ((round & 1) ? G - 1 - w : w);
    return j < plan.items ? j : -1;
  };
  // this round's item (s < 0: none), and the next one, whose first loads the
  // current item issues
  int s = -1, part = 0;
  if (compact) {
    const int64_t j = item_of(0);
    if (j >= 0) locate((int)j, s, part);
  } else {
    part = w / a.num_seqs;
    s = (w % a.num_seqs + a.num_seqs - part % a.num_seqs) % a.num_seqs;
  }
  for (int round = 0; s >= 0; ++round) {
    int s_next = -1, part_next = 0;
    if (compact) {
      const int64_t jn = item_of(round + 1);
      if (jn >= 0) locate((int)jn, s_next, part_next);
    }
    s = __builtin_amdgcn_readfirstlane(s);
    part = __builtin_amdgcn_readfirstlane(part);
    s_next = __builtin_amdgcn_readfirstlane(s_next);
    part_next = __builtin_amdgcn_readfirstlane(part_next);
    if (round > 0) __syncthreads();  // the previous item's merge has read every wave's LDS
    // An opaque copy of the thread index: lane-derived addresses are then
    // recomputed per item instead of being hoisted out of the item loop and
    // held in registers through the tile loop.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    // prefix partition length (shared mode): the plan's, or the host's minimum
    // shared mode: a description is checked only by the longest-first plan,
    // which the host always picks for one-launch shared calls
    decode_item<T, D, GT, F8, MODE, HP>(a, smem, tid, unit, s, part, compact ? plan.p_pre : a.prefix_partition_tokens,
                                    !compact || plan.bad_desc, hd, s_next, part_next);
    s = s_next;
    part = part_next;
  }
}

// Merge of the partition partials of a split sequence (one workgroup per
// sequence and query head):
//   M = max_p m_p,  out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p
// Thread (d, grp) folds partitions grp, grp + kGroups, ... for dimension d
// with the same online rescaling as the decode kernel (four partitions per
// step, loads issued together); the kGroups partial states are then combined
// in LDS.
constexpr int kReduceThreads = 1024;

template <typename T, int D>
__global__ __launch_bounds__(kReduceThreads) void paged_decode_reduce_kernel(DecodeArgs a) {
  constexpr int kGroups = kReduceThreads / D;
  __shared__ float red_num[kGroups][D];
  __shared__ float2 red_ml[kGroups];
  __shared__ int red_bad[kGroups];
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int L = a.seq_lens[s];
  const int P = a.partition_tokens;
  // suffix mode (shared-prefix decode): partitions start after the prefix
  const int tok0 = a.prefix_lens ? a.prefix_lens[s] : 0;
  if (tok0 < 0 || (tok0 & (a.block_size - 1)) != 0 || L - tok0 <= P ||
      (int64_t)L > (int64_t)a.max_blocks * a.block_size)
    return;  // single partition or invalid
  const int nparts = (L - tok0 + P - 1) / P;
  const int d = threadIdx.x % D;
  const int grp = threadIdx.x / D;
  const int64_t row = (int64_t)s * a.n_heads + h;
  const float2 *ml = a.part_ml + row * a.max_parts;
  const float *acc = a.part_acc + row * a.max_parts * D + d;
  float M = -INFINITY, num = 0.f, den = 0.f;
  bool bad = false;
  int p = grp;
  for (; p + 3 * kGroups < nparts; p += 4 * kGroups) {
    float2 v[4];
    float x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      v[u] = ml[p + u * kGroups];
      x[u] = acc[(int64_t)(p + u * kGroups) * D];
    }
    float mn = M;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      bad |= v[u].x != v[u].x;
      mn = fmaxf(mn, v[u].x);
    }
    const float f0 = __builtin_amdgcn_exp2f(M - mn);  // 0 while M = -inf
    num *= f0;
    den *= f0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float f = __builtin_amdgcn_exp2f(v[u].x - mn);
      den = fmaf(f, v[u].y, den);
      num = fmaf(f, x[u], num);
    }
    M = mn;
  }
  for (; p < nparts; p += kGroups) {
    const float2 v = ml[p];
    bad |= v.x != v.x;
    const float mn = fmaxf(M, v.x);
    const float f0 = __builtin_amdgcn_exp2f(M - mn);
    const float f = __builtin_amdgcn_exp2f(v.x - mn);
    den = fmaf(f, v.y, den * f0);
    num = fmaf(f, acc[(int64_t)p * D], num * f0);
    M = mn;
  }
  red_num[grp][d] = num;
  if (d == 0) {
    red_ml[grp] = make_float2(M, den);
    red_bad[grp] = bad;
  }
  __syncthreads();
  if (grp == 0) {
    float Mt = -INFINITY;
    int any_bad = 0;
#pragma unroll
    for (int g2 = 0; g2 < kGroups; ++g2) {
      Mt = fmaxf(Mt, red_ml[g2].x);
      any_bad |= red_bad[g2];
    }
    float nt = 0.f, dt = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < kGroups; ++g2) {
      const float2 v = red_ml[g2];
      const float f = v.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(v.x - Mt);  // empty groups
      dt = fmaf(f, v.y, dt);
      nt = fmaf(f, red_num[g2][d], nt);
    }
    float o = any_bad ? __builtin_nanf("") : nt / dt;
    if (tok0 > 0 && !any_bad) o = fold_partial(Mt, nt, dt, a.pre_ml[row], a.pre_acc[row * D + d]);
    static_cast<T *>(a.out)[row * D + d] = static_cast<T>(o);
  }
}

// The same merge when the table width allows at most kFewParts partitions:
// one thread per output element (query head, dimension) of kMergeHeadsPerThread
// heads, every partial of those elements loaded at once and then combined.
// A workgroup of kMergeThreads covers kMergeThreads / D * kMergeHeadsPerThread
// heads of one sequence; workgroups of unsplit sequences return after reading
// the length.
constexpr int kFewParts = 8;
constexpr int kMergeThreads = 256;
constexpr int kMergeHeadsPerThread = 4;

template <int D> __host__ __device__ constexpr int merge_heads_per_wg() {
  return kMergeThreads / D * kMergeHeadsPerThread;
}

template <typename T, int D>
__global__ __launch_bounds__(kMergeThreads) void paged_decode_merge_few_kernel(DecodeArgs a) {
  constexpr int kHL = kMergeThreads / D;  // head lanes per workgroup
  constexpr int kHPT = kMergeHeadsPerThread;
  constexpr int kHW = merge_heads_per_wg<D>();
  const int hblocks = (a.n_heads + kHW - 1) / kHW;
  const int s = blockIdx.x / hblocks;
  const int hb = blockIdx.x - s * hblocks;
  const int L = a.seq_lens[s];
  const int P = a.partition_tokens;
  const int tok0 = a.prefix_lens ? a.prefix_lens[s] : 0;  // suffix mode
  if (tok0 < 0 || (tok0 & (a.block_size - 1)) != 0 || L - tok0 <= P ||
      (int64_t)L > (int64_t)a.max_blocks * a.block_size)
    return;  // single partition or invalid
  const int nparts = (L - tok0 + P - 1) / P;  // 2 .. max_parts <= kFewParts
  const int d = threadIdx.x % D;
  const int hl = threadIdx.x / D;
  float2 ml[kHPT][kFewParts];
  float x[kHPT][kFewParts];
#pragma unroll
  for (int j = 0; j < kHPT; ++j) {
    const int h = hb * kHW + j * kHL + hl;
    const int64_t row = ((int64_t)s * a.n_heads + h) * a.max_parts;
#pragma unroll
    for (int p = 0; p < kFewParts; ++p) {
      if (h < a.n_heads && p < nparts) {
        ml[j][p] = a.part_ml[row + p];
        x[j][p] = a.part_acc[(row + p) * D + d];
      } else {
        ml[j][p] = make_float2(-INFINITY, 0.f);
        x[j][p] = 0.f;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < kHPT; ++j) {
    const int h = hb * kHW + j * kHL + hl;
    if (h >= a.n_heads) continue;
    float M = -INFINITY;
    bool bad = false;
#pragma unroll
    for (int p = 0; p < kFewParts; ++p) {
      bad |= ml[j][p].x != ml[j][p].x;
      M = fmaxf(M, ml[j][p].x);
    }
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int p = 0; p < kFewParts; ++p) {
      const float f = ml[j][p].x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml[j][p].x - M);
      den = fmaf(f, ml[j][p].y, den);
      num = fmaf(f, x[j][p], num);
    }
    const int64_t row = (int64_t)s * a.n_heads + h;
    float o = bad ? __builtin_nanf("") : num / den;
    if (tok0 > 0 && !bad) o = fold_partial(M, num, den, a.pre_ml[row], a.pre_acc[row * D + d]);
    static_cast<T *>(a.out)[row * D + d] = static_cast<T>(o);
  }
}

// Merge of split chunk-row items when a table allows more partitions than the
// in-kernel merge takes: one workgroup per (sequence, unit); thread t folds
// the partitions of output elements t, t + 256, ... of the item's rows with
// the same online rescaling (partitions that saw none of a row's tokens hold
// m = -inf and are skipped).
constexpr int kChunkReduceThreads = 256;

template <typename T, int D, int MODE>
__global__ __launch_bounds__(kChunkReduceThreads) void paged_chunk_reduce_kernel(DecodeArgs a) {
  static_assert(MODE == kModeChunk || MODE == kModePrefix, "rows modes");
  constexpr int kRows = 16;
  const int units = a.n_kv_heads * a.head_chunks;
  const int s = (int)(blockIdx.x / (unsigned)units);
  const int unit = (int)(blockIdx.x - (unsigned)s * units);
  const int g = unit / a.head_chunks;
  const int row0 = (unit - g * a.head_chunks) * kRows;
  const int G = a.group;
  const int q0 = a.query_start_loc[s];
  const int nq = a.query_start_loc[s + 1] - q0;
  if (q0 < 0 || (MODE == kModePrefix && (nq < 1 || q0 + nq > a.member_seqs))) return;
  const int L = MODE == kModePrefix ? a.prefix_lens[q0] : a.seq_lens[s];
  const int nh = max(0, min(kRows, nq * G - row0));
  if (nh == 0 || (int64_t)L > (int64_t)a.max_blocks * a.block_size) return;
  if (MODE == kModeChunk && L < nq) return;
  if (MODE == kModePrefix && (L <= 0 || (L & (a.block_size - 1)) != 0)) return;
  const int ctx = MODE == kModeChunk ? L - nq + (row0 + nh - 1) / G + 1 : L;
  const int P = a.partition_tokens;
  const int nparts = (ctx + P - 1) / P;
  if (nparts <= 1) return;  // written by the attention kernel
  for (int idx = threadIdx.x; idx < nh * D; idx += kChunkReduceThreads) {
    const int i = idx / D;
    const int d = idx - i * D;
    const int64_t prow = ((int64_t)s * units + unit) * kRows + i;
    const float2 *ml = a.part_ml + prow * a.max_parts;
    const float *acc = a.part_acc + prow * a.max_parts * D + d;
    float M = -INFINITY, num = 0.f, den = 0.f;
    bool bad = false;
    for (int p = 0; p < nparts; ++p) {
      const float2 v = ml[p];
      const float x = acc[(int64_t)p * D];
      bad |= v.x != v.x;
      if (!(v.x > -INFINITY)) continue;
      const float mn = fmaxf(M, v.x);
      const float f0 = __builtin_amdgcn_exp2f(M - mn);  // 0 while M = -inf
      const float f = __builtin_amdgcn_exp2f(v.x - mn);
      den = fmaf(f, v.y, den * f0);
      num = fmaf(f, x, num * f0);
      M = mn;
    }
    const int r = row0 + i;
    const int64_t orow = (int64_t)(q0 + r / G) * a.n_heads + g * G + r % G;
    if constexpr (MODE == kModePrefix) {
      a.pre_acc[orow * D + d] = bad ? __builtin_nanf("") : num;
      if (d == 0) a.pre_ml[orow] = make_float2(bad ? __builtin_nanf("") : M, den);
    } else {
      static_cast<T *>(a.out)[orow * D + d] = static_cast<T>(bad ? __builtin_nanf("") : num / den);
    }
  }
}

}  // namespace

// Compute units of the current device (cached per device).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

namespace {

// Decode workgroups per unit in the longest-first mode: at least one per
// sequence and enough for kWgsPerSlot rounds of the chip's resident slots,
// never more than the unit's largest possible item count.
constexpr int kWgsPerSlot = 2;

// The longest-first order of make_plan, built on the host from the host
// copy of the lengths: the full partitions (sequence-major), then the last
// partitions by decreasing length, in sequence order among equals. exact:
// by their exact length, where make_plan takes kRemBuckets buckets (with
// one item per workgroup the exact order measured faster; FP8 pools, whose
// workgroups walk two items, keep the buckets). With ticket claimers every
// workgroup must take one item (no more items per unit than workgroups).
// Leaves hp_items at zero, and the kernel on its own plan, when the order
// does not fit the arguments.
void host_plan(DecodeArgs &a, bool exact) {
  const int B = a.num_seqs;
  const int P = a.partition_tokens;
  const int64_t max_tok = (int64_t)a.max_blocks * a.block_size;
  if (B > kHostPlanSeqs || P < 1) return;
  int full[kHostPlanSeqs], key[kHostPlanSeqs], order[kHostPlanSeqs];
  int64_t items = B;
  for (int s = 0; s < B; ++s) {
    const int L = a.host_seq_lens[s];
    const bool ok = L > 0 && (int64_t)L <= max_tok;
    full[s] = ok ? (L - 1) / P : 0;
    if (full[s] + 1 > 255) return;  // partition ids take 8 bits
    const int shortfall = P - (L - full[s] * P);  // 0 .. P - 1 when ok
    key[s] = !ok ? INT_MAX : exact ? shortfall : (int)((int64_t)shortfall * kRemBuckets / P);
    order[s] = s;
    items += full[s];
  }
  if (items > kHostPlanItems || (a.tickets && items > a.wgs_per_unit)) return;
  int n = 0;
  for (int s = 0; s < B; ++s) {
    for (int p = 0; p < full[s]; ++p) a.hp[n++] = (uint16_t)(s | (p << 8));
    a.hp_np[s] = (uint8_t)(full[s] + 1);
  }
  std::stable_sort(order, order + B, [&](int x, int y) { return key[x] < key[y]; });
  for (int i = 0; i < B; ++i) a.hp[n++] = (uint16_t)(order[i] | (full[order[i]] << 8));
  a.hp_items = n;
}

template <typename T, int D, int GT, bool F8, int MODE = kModeDecode>
hipError_t launch_t(const DecodeArgs &args, hipStream_t stream) {
  DecodeArgs a = args;
  const int64_t units = (int64_t)a.n_kv_heads * a.head_chunks;
  const int64_t max_items = (int64_t)a.num_seqs * a.max_parts;
  if (compact_plan(a)) {
    static const int per_cu = [] {
      int nb = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, paged_decode_kernel<T, D, GT, F8, MODE>, kDecodeWaves * 64, 0) !=
              hipSuccess || nb <= 0)
        nb = 1;
      return nb;
    }();
    const int64_t resident = (int64_t)per_cu * device_cus();
    // FP8 pools (4 workgroups per CU): one round of resident slots measured
    // best (GQA batch 128: 40.2 -> 39.1 us against two)
    const int64_t slots = F8 ? resident : resident * kWgsPerSlot;
    int64_t g = (slots + units - 1) / units;
    // Tickets (the first `resident` workgroups keep their places, the rest
    // claim theirs) pay off when most workgroups take a single item: measured
    // on batches with more workgroups per unit than sequences and at least 32
    // sequences (GQA batch 128: -1.6 us); with fewer workgroups per unit
    // (MHA batch 64) or few long sequences (4 x 32K-128K), where workgroups
    // take two or more items, the claims cost 0.5-1% and tickets stay off.
    // FP8 pools (4 workgroups per CU, half the bytes per item) measured
    // slower with tickets (GQA batch 128: 40.2 -> 43.0 us): off as well.
    if (F8 || g <= a.num_seqs || a.num_seqs < 32) a.tickets = nullptr;
    if (g < a.num_seqs) g = a.num_seqs;
    a.wgs_per_unit = (int32_t)(g < max_items ? g : max_items);
    a.static_wgs = (int32_t)std::min<int64_t>(resident, units * a.wgs_per_unit);
    if (a.static_wgs >= units * a.wgs_per_unit) a.tickets = nullptr;
  } else {
    a.wgs_per_unit = (int32_t)max_items;
    a.tickets = nullptr;
  }
  a.hp_items = 0;
  // 16-bit pools: only where ticket claimers place every item (one item per
  // workgroup); FP8 pools (no tickets, a workgroup may take two items): always
  if constexpr (MODE == kModeAppend) {
    if (a.host_seq_lens && (a.tickets || F8)) host_plan(a, !F8);
  }
  dim3 grid((unsigned)(units * a.wgs_per_unit), 1, 1);
  if constexpr (MODE == kModeAppend) {
    if (a.hp_items > 0)
      hipLaunchKernelGGL((paged_decode_kernel<T, D, GT, F8, MODE, true>), grid, dim3(kDecodeWaves * 64), 0, stream,
                         a);
    else
      hipLaunchKernelGGL((paged_decode_kernel<T, D, GT, F8, MODE>), grid, dim3(kDecodeWaves * 64), 0, stream, a);
  } else {
    hipLaunchKernelGGL((paged_decode_kernel<T, D, GT, F8, MODE>), grid, dim3(kDecodeWaves * 64), 0, stream, a);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.max_parts == 1 || a.arrivals != nullptr) return err;
  if constexpr (MODE == kModeChunk || MODE == kModePrefix) {
    hipLaunchKernelGGL((paged_chunk_reduce_kernel<T, D, MODE>), dim3((unsigned)(units * a.num_seqs)),
                       dim3(kChunkReduceThreads), 0, stream, a);
    return hipGetLastError();
  }
  if (a.max_parts <= kFewParts) {
    const int hblocks = (a.n_heads + merge_heads_per_wg<D>() - 1) / merge_heads_per_wg<D>();
    hipLaunchKernelGGL((paged_decode_merge_few_kernel<T, D>), dim3((unsigned)(a.num_seqs * hblocks)),
                       dim3(kMergeThreads), 0, stream, a);
  } else {
    dim3 rgrid(a.n_heads, a.num_seqs, 1);
    hipLaunchKernelGGL((paged_decode_reduce_kernel<T, D>), rgrid, dim3(kReduceThreads), 0, stream, a);
  }
  return hipGetLastError();
}

template <typename T, bool F8>
hipError_t launch_rows_t(int head_dim, const DecodeArgs &a, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_t<T, 64, 16, F8, kModeChunk>(a, stream);
    case 128: return launch_t<T, 128, 16, F8, kModeChunk>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int D, bool F8>
hipError_t launch_d(int gt, const DecodeArgs &a, hipStream_t stream) {
  switch (gt) {
    case 1: return launch_t<T, D, 1, F8>(a, stream);
    case 2: return launch_t<T, D, 2, F8>(a, stream);
    case 4: return launch_t<T, D, 4, F8>(a, stream);
    case 8: return launch_t<T, D, 8, F8>(a, stream);
    case 16: return launch_t<T, D, 16, F8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, bool F8>
hipError_t launch_dt(int head_dim, int gt, const DecodeArgs &a, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_d<T, 64, F8>(gt, a, stream);
    case 128: return launch_d<T, 128, F8>(gt, a, stream);
    default: return hipErrorInvalidValue;
  }
}

__global__ void zero_i32_kernel(int32_t *p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

}  // namespace

hipError_t launch_zero_i32(int32_t *p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(zero_i32_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0,
                     stream, p, n);
  return hipGetLastError();
}

bool decode_compact_plan(const DecodeArgs &a) { return compact_plan(a); }

int decode_head_tile(int group) {
  int gt = 1;
  while (gt < group && gt < 16) gt <<= 1;
  return gt;
}

hipError_t launch_decode(DType dt, int head_dim, const DecodeArgs &a, hipStream_t stream) {
  const int gt = decode_head_tile(a.group);
  switch (dt) {
    case DType::F32: return launch_dt<float, false>(head_dim, gt, a, stream);
    case DType::F16: return launch_dt<_Float16, false>(head_dim, gt, a, stream);
    case DType::BF16: return launch_dt<__bf16, false>(head_dim, gt, a, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_rows(DType dt, int head_dim, bool fp8, const DecodeArgs &a, hipStream_t stream) {
  switch (dt) {
    case DType::F16: return fp8 ? launch_rows_t<_Float16, true>(head_dim, a, stream)
                                : launch_rows_t<_Float16, false>(head_dim, a, stream);
    case DType::BF16: return fp8 ? launch_rows_t<__bf16, true>(head_dim, a, stream)
                                 : launch_rows_t<__bf16, false>(head_dim, a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int D, bool F8>
hipError_t launch_shared_prefix_td(int gt, const DecodeArgs &pre, const DecodeArgs &suf, hipStream_t stream) {
  hipError_t e = launch_t<T, D, 16, F8, kModePrefix>(pre, stream);
  if (e != hipSuccess) return e;
  switch (gt) {
    case 1: return launch_t<T, D, 1, F8, kModeSuffix>(suf, stream);
    case 2: return launch_t<T, D, 2, F8, kModeSuffix>(suf, stream);
    case 4: return launch_t<T, D, 4, F8, kModeSuffix>(suf, stream);
    case 8: return launch_t<T, D, 8, F8, kModeSuffix>(suf, stream);
    case 16: return launch_t<T, D, 16, F8, kModeSuffix>(suf, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, bool F8>
hipError_t launch_shared_fused_t(int head_dim, const DecodeArgs &a, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_t<T, 64, 16, F8, kModeShared>(a, stream);
    case 128: return launch_t<T, 128, 16, F8, kModeShared>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, bool F8>
hipError_t launch_shared_prefix_t(int head_dim, int gt, const DecodeArgs &pre, const DecodeArgs &suf,
                                  hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_shared_prefix_td<T, 64, F8>(gt, pre, suf, stream);
    case 128: return launch_shared_prefix_td<T, 128, F8>(gt, pre, suf, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_shared_prefix(DType dt, int head_dim, bool fp8, const DecodeArgs &pre, const DecodeArgs &suf,
                                hipStream_t stream) {
  const int gt = decode_head_tile(suf.group);
  switch (dt) {
    case DType::F16: return fp8 ? launch_shared_prefix_t<_Float16, true>(head_dim, gt, pre, suf, stream)
                                : launch_shared_prefix_t<_Float16, false>(head_dim, gt, pre, suf, stream);
    case DType::BF16: return fp8 ? launch_shared_prefix_t<__bf16, true>(head_dim, gt, pre, suf, stream)
                                 : launch_shared_prefix_t<__bf16, false>(head_dim, gt, pre, suf, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_shared_fused(DType dt, int head_dim, bool fp8, const DecodeArgs &a, hipStream_t stream) {
  switch (dt) {
    case DType::F16: return fp8 ? launch_shared_fused_t<_Float16, true>(head_dim, a, stream)
                                : launch_shared_fused_t<_Float16, false>(head_dim, a, stream);
    case DType::BF16: return fp8 ? launch_shared_fused_t<__bf16, true>(head_dim, a, stream)
                                 : launch_shared_fused_t<__bf16, false>(head_dim, a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int D, bool F8>
hipError_t launch_append_td(int gt, const DecodeArgs &a, hipStream_t stream) {
  switch (gt) {
    case 1: return launch_t<T, D, 1, F8, kModeAppend>(a, stream);
    case 2: return launch_t<T, D, 2, F8, kModeAppend>(a, stream);
    case 4: return launch_t<T, D, 4, F8, kModeAppend>(a, stream);
    case 8: return launch_t<T, D, 8, F8, kModeAppend>(a, stream);
    case 16: return launch_t<T, D, 16, F8, kModeAppend>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, bool F8>
hipError_t launch_append_t(int head_dim, int gt, const DecodeArgs &a, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_append_td<T, 64, F8>(gt, a, stream);
    case 128: return launch_append_td<T, 128, F8>(gt, a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_append(DType dt, int head_dim, bool fp8, const DecodeArgs &a, hipStream_t stream) {
  const int gt = decode_head_tile(a.group);
  switch (dt) {
    case DType::F16:
      return fp8 ? launch_append_t<_Float16, true>(head_dim, gt, a, stream)
                 : launch_append_t<_Float16, false>(head_dim, gt, a, stream);
    case DType::BF16:
      return fp8 ? launch_append_t<__bf16, true>(head_dim, gt, a, stream)
                 : launch_append_t<__bf16, false>(head_dim, gt, a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_fp8(DType dt, int head_dim, const DecodeArgs &a, hipStream_t stream) {
  const int gt = decode_head_tile(a.group);
  switch (dt) {
    case DType::F16: return launch_dt<_Float16, true>(head_dim, gt, a, stream);
    case DType::BF16: return launch_dt<__bf16, true>(head_dim, gt, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
