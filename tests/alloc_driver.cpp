// Test driver for the host block allocator (kvs_alloc_* in csrc/alloc.cpp), built on the host
// with AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_alloc_sanitized.py.
//
// Reads one operation per line from stdin and prints one result line per operation:
//   create N [b0 b1 ...]   -> "rc"            (free order given when ids follow; else 0..N-1)
//   alloc                  -> "rc block"
//   incref B | decref B    -> "rc"
//   cow B                  -> "rc block copied"
//   count B                -> "rc"            (the count, or a negative code)
//   nfree                  -> "rc"
//   freelist               -> "rc b0 b1 ..."  (rc = number of ids written)
//   destroy                -> "0"
// Error messages go through kvs::fail, defined here so the allocator links without the HIP
// runtime.
#include <cstdarg>
#include <cstdio>
#include <iostream>
#include <sstream>
#include <string>
#include <vector>

#include "kvs.h"

namespace kvs {
int fail(int code, const char* fmt, ...) {
  char buf[256];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  return code;
}
}  // namespace kvs

int main() {
  kvs_alloc* a = nullptr;
  std::string line;
  while (std::getline(std::cin, line)) {
    std::istringstream in(line);
    std::string op;
    in >> op;
    if (op == "create") {
      int n = 0;
      in >> n;
      std::vector<int32_t> order;
      int32_t b;
      bool given = false;
      while (in >> b) {
        order.push_back(b);
        given = true;
      }
      if (a) kvs_alloc_destroy(a);
      a = nullptr;
      int rc = kvs_alloc_create(n, given ? order.data() : nullptr, (int)order.size(), &a);
      std::printf("%d\n", rc);
    } else if (op == "alloc") {
      int32_t out = -1;
      int rc = kvs_alloc_block(a, &out);
      std::printf("%d %d\n", rc, rc == KVS_OK ? out : -1);
    } else if (op == "incref" || op == "decref" || op == "count") {
      int32_t b = 0;
      in >> b;
      int rc = op == "incref" ? kvs_alloc_incref(a, b) : op == "decref" ? kvs_alloc_decref(a, b)
                                                                        : kvs_alloc_refcount(a, b);
      std::printf("%d\n", rc);
    } else if (op == "cow") {
      int32_t b = 0, out = -1;
      int copied = -1;
      in >> b;
      int rc = kvs_alloc_cow(a, b, &out, &copied);
      std::printf("%d %d %d\n", rc, rc == KVS_OK ? out : -1, rc == KVS_OK ? copied : -1);
    } else if (op == "nfree") {
      std::printf("%d\n", kvs_alloc_num_free(a));
    } else if (op == "freelist") {
      int n = kvs_alloc_num_free(a);
      std::vector<int32_t> buf(n > 0 ? n : 1);
      int m = kvs_alloc_free_list(a, buf.data(), n);
      std::printf("%d", m);
      for (int i = 0; i < m; ++i) std::printf(" %d", buf[i]);
      std::printf("\n");
    } else if (op == "destroy") {
      kvs_alloc_destroy(a);
      a = nullptr;
      std::printf("0\n");
    }
  }
  if (a) kvs_alloc_destroy(a);
  return 0;
}
