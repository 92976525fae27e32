// Host-side check of the packed-batch work order: reads
//   mode causal tile fkv bq nseq  lq_0 lk_0 ... lq_{n-1} lk_{n-1}
// from stdin, builds the item list with the scheduler's own item, cost and
// sort-key functions, sorts the keys ascending (as the device sort does) and
// prints one "seq idx cost" line per item in the resulting order (a split
// forward chunk prints its index as -(chunk + 1)).
#include <algorithm>
#include <cstdio>
#include <vector>

#include "../../exact_attention_80_amd/csrc/fa_sched_keys.h"

int main() {
  int mode, causal, tile, fkv, bq, nseq;
  if (std::scanf("%d %d %d %d %d %d", &mode, &causal, &tile, &fkv, &bq, &nseq) != 6) return 1;
  std::vector<int> cu_q(nseq + 1, 0), cu_k(nseq + 1, 0);
  for (int s = 0; s < nseq; ++s) {
    int lq, lk;
    if (std::scanf("%d %d", &lq, &lk) != 2) return 1;
    cu_q[s + 1] = cu_q[s] + lq;
    cu_k[s + 1] = cu_k[s] + lk;
  }
  using namespace fa::sched;
  std::vector<unsigned long long> keys;
  for (int s = 0; s < nseq; ++s) {
    const int lq = cu_q[s + 1] - cu_q[s], lk = cu_k[s + 1] - cu_k[s];
    const int nt = seq_items(mode, causal != 0, cu_q.data(), cu_k.data(), s, tile, fkv);
    // the cost the scheduler kernel passes: modes 0, 2 the sequence's largest
    // tile cost, mode 1 the tile's own
    int seq_cost = 0;
    for (int k = 0; k < nt; ++k)
      seq_cost = imax(seq_cost, item_cost(mode, causal != 0, lq, lk, tile,
                                          seq_item_index(mode, causal != 0, lq, lk, tile, fkv, k),
                                          fkv, bq));
    for (int k = 0; k < nt; ++k) {
      const int idx = seq_item_index(mode, causal != 0, lq, lk, tile, fkv, k);
      const int cost = mode == 1 ? item_cost(mode, causal != 0, lq, lk, tile, idx, fkv, bq) : seq_cost;
      keys.push_back(sort_key(mode, cost, s, idx));
    }
  }
  std::sort(keys.begin(), keys.end());
  for (unsigned long long k : keys) {
    int seq, idx;
    decode_key(mode, k, seq, idx);
    const int lq = cu_q[seq + 1] - cu_q[seq], lk = cu_k[seq + 1] - cu_k[seq];
    const int cost = item_cost(mode, causal != 0, lq, lk, tile, idx, fkv, bq);
    const int shown = (idx & fa::kSplitItem) ? -((idx & 0xFFFFF) + 1) : idx;
    std::printf("%d %d %d\n", seq, shown, cost);
  }
  return 0;
}
