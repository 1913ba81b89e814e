// Host block allocator of the paged KV cache.
//
// [PAG] Ultralytics glossary, "PagedAttention", "How paging works": a request takes a new
// block only when its last block is full, from wherever a free block is; the worked example
// pops free blocks from the front of a list.  "Sharing blocks between sequences": one
// reference count per block and copy-on-write before writing a shared block.  "Related
// techniques" (continuous batching): a finished sequence's blocks go back to the free pool
// at once.
//
// The free list is a ring buffer of capacity num_blocks used first-in first-out: allocation
// pops the front, a block whose count drops to zero is pushed at the back.  Every operation
// is O(1); nothing here touches the device.
#include <cstdint>
#include <new>
#include <vector>

#include "kvs.h"

namespace kvs {
int fail(int code, const char* fmt, ...);
}

struct kvs_alloc {
  int32_t n = 0;
  std::vector<int32_t> ref;    // reference count per block, 0 = free
  std::vector<int32_t> ring;   // free list storage
  int32_t head = 0;            // index of the front
  int32_t size = 0;            // number of free blocks

  void push_back(int32_t b) {
    ring[(head + size) % n] = b;
    ++size;
  }
  int32_t pop_front() {
    int32_t b = ring[head];
    head = (head + 1) % n;
    --size;
    return b;
  }
};

extern "C" int kvs_alloc_create(int num_blocks, const int32_t* initial_free_order, int n_initial,
                                kvs_alloc** out) {
  if (!out) return kvs::fail(KVS_E_INVAL, "kvs_alloc_create: out is NULL");
  *out = nullptr;
  if (num_blocks <= 0) return kvs::fail(KVS_E_INVAL, "kvs_alloc_create: num_blocks must be > 0");
  kvs_alloc* a = new (std::nothrow) kvs_alloc;
  if (!a) return kvs::fail(KVS_E_INVAL, "kvs_alloc_create: out of host memory");
  a->n = num_blocks;
  a->ref.assign(num_blocks, 0);
  a->ring.assign(num_blocks, 0);
  if (!initial_free_order) {
    for (int32_t b = 0; b < num_blocks; ++b) a->push_back(b);
  } else {
    if (n_initial < 0 || n_initial > num_blocks) {
      delete a;
      return kvs::fail(KVS_E_INVAL, "kvs_alloc_create: n_initial out of range");
    }
    std::vector<char> seen(num_blocks, 0);
    for (int i = 0; i < n_initial; ++i) {
      int32_t b = initial_free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete a;
        return kvs::fail(KVS_E_INVAL, "kvs_alloc_create: free order must hold distinct ids in range");
      }
      seen[b] = 1;
      a->push_back(b);
    }
    for (int32_t b = 0; b < num_blocks; ++b)
      if (!seen[b]) a->ref[b] = 1;   // not listed: starts in use
  }
  *out = a;
  return KVS_OK;
}

extern "C" void kvs_alloc_destroy(kvs_alloc* a) { delete a; }

extern "C" int kvs_alloc_block(kvs_alloc* a, int32_t* out_block) {
  if (!a || !out_block) return kvs::fail(KVS_E_INVAL, "kvs_alloc_block: NULL argument");
  if (a->size == 0) return kvs::fail(KVS_E_NOBLOCKS, "kvs_alloc_block: no free block");
  int32_t b = a->pop_front();
  a->ref[b] = 1;
  *out_block = b;
  return KVS_OK;
}

extern "C" int kvs_alloc_incref(kvs_alloc* a, int32_t block) {
  if (!a || block < 0 || block >= a->n) return kvs::fail(KVS_E_INVAL, "kvs_alloc_incref: bad block %d", block);
  if (a->ref[block] == 0) return kvs::fail(KVS_E_STATE, "kvs_alloc_incref: block %d is free", block);
  ++a->ref[block];
  return KVS_OK;
}

extern "C" int kvs_alloc_decref(kvs_alloc* a, int32_t block) {
  if (!a || block < 0 || block >= a->n) return kvs::fail(KVS_E_INVAL, "kvs_alloc_decref: bad block %d", block);
  if (a->ref[block] == 0) return kvs::fail(KVS_E_STATE, "kvs_alloc_decref: block %d is already free", block);
  if (--a->ref[block] == 0) a->push_back(block);
  return KVS_OK;
}

extern "C" int kvs_alloc_refcount(const kvs_alloc* a, int32_t block) {
  if (!a || block < 0 || block >= a->n) return kvs::fail(KVS_E_INVAL, "kvs_alloc_refcount: bad block %d", block);
  return a->ref[block];
}

extern "C" int kvs_alloc_num_free(const kvs_alloc* a) {
  if (!a) return kvs::fail(KVS_E_INVAL, "kvs_alloc_num_free: NULL allocator");
  return a->size;
}

extern "C" int kvs_alloc_free_list(const kvs_alloc* a, int32_t* out, int cap) {
  if (!a || (!out && cap > 0) || cap < 0) return kvs::fail(KVS_E_INVAL, "kvs_alloc_free_list: bad argument");
  int m = a->size < cap ? a->size : cap;
  for (int i = 0; i < m; ++i) out[i] = a->ring[(a->head + i) % a->n];
  return m;
}

extern "C" int kvs_alloc_cow(kvs_alloc* a, int32_t block, int32_t* out_block, int* copied) {
  if (!a || !out_block || !copied || block < 0 || block >= a->n)
    return kvs::fail(KVS_E_INVAL, "kvs_alloc_cow: bad argument");
  if (a->ref[block] == 0) return kvs::fail(KVS_E_STATE, "kvs_alloc_cow: block %d is free", block);
  if (a->ref[block] == 1) {
    *out_block = block;
    *copied = 0;
    return KVS_OK;
  }
  if (a->size == 0) return kvs::fail(KVS_E_NOBLOCKS, "kvs_alloc_cow: no free block");
  int32_t nb = a->pop_front();
  a->ref[nb] = 1;
  --a->ref[block];   // still > 0: the other sharers keep it
  *out_block = nb;
  *copied = 1;
  return KVS_OK;
}
