// CPU harness for the header-only cache plan: reads commands on stdin and
// prints the resident set after each one.
//   first line: n_sink n_local
//   then: "a <n_frames> <t0>" (append) or "r" (reset)
// output line per command: <code> <n_appended> [frame,t,segment,slot ...]
// code 0 = applied, 1/2/3 = rejected by check_append, 9 = planned slot not resident.
#include <cstdio>
#include <iostream>
#include <string>

#include "cache_plan.hpp"

int main() {
  int ns = 0, nl = 0;
  if (!(std::cin >> ns >> nl)) return 2;
  sa::CachePlan plan(ns, nl);
  std::string cmd;
  while (std::cin >> cmd) {
    int code = 0;
    if (cmd == "a") {
      int n = 0;
      long long t0 = 0;
      std::cin >> n >> t0;
      code = plan.check_append(n, t0);
      if (code == 0) {
        const auto planned = plan.plan_append(n, t0);
        plan.commit_append(n, t0);
        const auto res = plan.resident();
        for (const auto& p : planned) {
          bool found = false;
          for (const auto& r : res)
            if (r.frame == p.frame && r.store_slot == p.store_slot && r.t == p.t && r.slot == p.slot &&
                r.segment == p.segment)
              found = true;
          if (!found) code = 9;
        }
      }
    } else if (cmd == "r") {
      plan.reset();
    } else {
      return 3;
    }
    std::printf("%d %lld", code, static_cast<long long>(plan.n_appended()));
    for (const auto& r : plan.resident())
      std::printf(" %lld,%lld,%d,%d", static_cast<long long>(r.frame), static_cast<long long>(r.t), r.segment,
                  r.slot);
    std::printf("\n");
  }
  return 0;
}
