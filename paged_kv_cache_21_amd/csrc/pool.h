// Host block pool state, shared by the pool's C ABI and the prefix cache, which
// holds references on the blocks it caches.
#pragma once

#include <cstdint>
#include <deque>
#include <unordered_map>
#include <vector>

struct pkv_pool {
  struct Seq {
    std::vector<int32_t> table;    // block ids; host slot ids where on_host[i] is set
    std::vector<uint8_t> on_host;  // swapped-out sequences only: entry i lives in a host slot
    bool swapped = false;
    int32_t len = 0;
  };
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> ref;          // references per block: sequences plus other holders
  std::deque<int32_t> free_list;     // FIFO: taken from the front, returned to the back
  std::unordered_map<int64_t, Seq> seqs;
  int32_t num_host_slots = 0;        // swap space: host slots, one block each
  std::deque<int32_t> host_free;     // FIFO like free_list

  // One more reference on an allocated block.
  void retain(int32_t b) { ref[b] += 1; }
  // One reference less; true when the block went back to the free list.
  bool release(int32_t b) {
    if (--ref[b] == 0) {
      free_list.push_back(b);
      return true;
    }
    return false;
  }
};
