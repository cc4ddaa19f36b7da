// Host helper of the shared-prefix decode (declared in pkv_shared_prefix.h):
// finds runs of consecutive sequences whose block tables start with the same
// physical blocks, as forks of one prompt do (vLLM paper page, block sharing
// for parallel sampling and beam search; vLLM notes page, ref_count sharing),
// and the number of whole blocks they share.
#include <stdint.h>

#include <algorithm>

#include "pkv_shared_prefix.h"
#include "status.h"

namespace {

// Whole blocks of sequence s that hold tokens only of s's length.
int32_t full_blocks(const int32_t *seq_lens, int32_t s, int32_t block_size) { return seq_lens[s] / block_size; }

}  // namespace

extern "C" int pkv_shared_prefix_groups(const int32_t *block_tables, const int32_t *seq_lens, int32_t num_seqs,
                                        int32_t max_blocks_per_seq, int32_t block_size, int32_t *group_start,
                                        int32_t *prefix_lens, int32_t *num_groups, int32_t *max_group_size) {
  if (num_seqs < 0 || max_blocks_per_seq < 1 || block_size < 1)
    return pkv::set_error(PKV_ERR_INVALID, "num_seqs must be >= 0, max_blocks_per_seq and block_size >= 1");
  if (!num_groups || (num_seqs > 0 && (!block_tables || !seq_lens || !group_start || !prefix_lens)))
    return pkv::set_error(PKV_ERR_INVALID, "null pointer");
  const int64_t cap = (int64_t)max_blocks_per_seq * block_size;
  for (int32_t s = 0; s < num_seqs; ++s)
    if (seq_lens[s] < 0 || seq_lens[s] > cap)
      return pkv::set_error(PKV_ERR_INVALID, "seq_lens[%d] = %d outside [0, %lld]", s, seq_lens[s], (long long)cap);
  int32_t groups = 0, largest = 0;
  int32_t s = 0;
  while (s < num_seqs) {
    const int32_t *first = block_tables + (int64_t)s * max_blocks_per_seq;
    // shared whole blocks of the group so far: all of the first member's
    int32_t shared = full_blocks(seq_lens, s, block_size);
    int32_t e = s + 1;
    while (e < num_seqs) {
      const int32_t *row = block_tables + (int64_t)e * max_blocks_per_seq;
      const int32_t limit = std::min(shared, full_blocks(seq_lens, e, block_size));
      int32_t k = 0;
      while (k < limit && row[k] == first[k]) ++k;
      if (k == 0) break;  // no common first block: a new group starts at e
      shared = k;
      ++e;
    }
    const int32_t size = e - s;
    const int32_t prefix = size > 1 ? shared * block_size : 0;
    group_start[groups++] = s;
    for (int32_t i = s; i < e; ++i) prefix_lens[i] = prefix;
    largest = std::max(largest, size);
    s = e;
  }
  if (num_seqs > 0) group_start[groups] = num_seqs;
  *num_groups = groups;
  if (max_group_size) *max_group_size = largest;
  return pkv::clear_error();
}
