// Command-script driver for the host page table, built with g++ under
// AddressSanitizer and UBSan by the CPU tests. Reads one command per line on
// stdin and prints one result line per command on stdout:
//
//   create N P T W PIN ORDER   ORDER = 0 (identity) or 1 (N ids follow on the line)
//   alloc CAP                  -> "alloc <status> <ids...>"
//   commit CAP                 -> "commit <status> <n> <ids...>"
//   export CAP                 -> "export <status> <n_chunks> <ids...>"
//   free                       -> "free <status> <n>"
//   ppc                        -> "ppc <status> <n>"
//   destroy
//
// CAP is the capacity passed to the call (int32 elements), so the tests can
// drive the error paths as well as the normal schedule.
#include <cstdint>
#include <cstdio>
#include <iostream>
#include <sstream>
#include <string>
#include <vector>

#include "wf_attn.h"

int main() {
  wf_page_table* pt = nullptr;
  std::string line;
  while (std::getline(std::cin, line)) {
    std::istringstream in(line);
    std::string cmd;
    if (!(in >> cmd)) continue;
    if (cmd == "create") {
      int32_t n, p, t, w, pin, ord;
      in >> n >> p >> t >> w >> pin >> ord;
      std::vector<int32_t> order;
      if (ord) {
        order.resize(size_t(n > 0 ? n : 0));
        for (auto& x : order) in >> x;
      }
      if (pt) wf_page_table_destroy(pt);
      pt = nullptr;
      const wf_status st =
          wf_page_table_create(n, p, t, w, pin, ord ? order.data() : nullptr, &pt);
      std::printf("create %d\n", st);
    } else if (cmd == "alloc") {
      int32_t cap;
      in >> cap;
      std::vector<int32_t> ids(size_t(cap > 0 ? cap : 0), -7);
      const wf_status st = wf_page_table_alloc_chunk(pt, cap > 0 ? ids.data() : nullptr, cap);
      std::printf("alloc %d", st);
      int32_t ppc = 0;
      if (st == WF_OK && wf_page_table_pages_per_chunk(pt, &ppc) == WF_OK)
        for (int32_t i = 0; i < ppc; ++i) std::printf(" %d", ids[size_t(i)]);
      std::printf("\n");
    } else if (cmd == "commit") {
      int32_t cap;
      in >> cap;
      std::vector<int32_t> ids(size_t(cap > 0 ? cap : 0), -7);
      int32_t n = -1;
      const wf_status st = wf_page_table_commit(pt, cap > 0 ? ids.data() : nullptr, cap, &n);
      std::printf("commit %d %d", st, n);
      if (st == WF_OK && cap > 0)
        for (int32_t i = 0; i < n; ++i) std::printf(" %d", ids[size_t(i)]);
      std::printf("\n");
    } else if (cmd == "export") {
      int32_t cap;
      in >> cap;
      std::vector<int32_t> ids(size_t(cap > 0 ? cap : 0), -7);
      int32_t n = -1, ppc = 0;
      const wf_status st = wf_page_table_export(pt, cap > 0 ? ids.data() : nullptr, cap, &n);
      std::printf("export %d %d", st, n);
      if (st == WF_OK && wf_page_table_pages_per_chunk(pt, &ppc) == WF_OK)
        for (int64_t i = 0; i < int64_t(n) * ppc; ++i) std::printf(" %d", ids[size_t(i)]);
      std::printf("\n");
    } else if (cmd == "free") {
      int32_t n = -1;
      const wf_status st = wf_page_table_num_free(pt, &n);
      std::printf("free %d %d\n", st, n);
    } else if (cmd == "ppc") {
      int32_t n = -1;
      const wf_status st = wf_page_table_pages_per_chunk(pt, &n);
      std::printf("ppc %d %d\n", st, n);
    } else if (cmd == "destroy") {
      wf_page_table_destroy(pt);
      pt = nullptr;
      std::printf("destroy\n");
    } else {
      std::printf("unknown %s\n", cmd.c_str());
      return 2;
    }
  }
  if (pt) wf_page_table_destroy(pt);
  return 0;
}
