// Places of the late decode workgroups.
//
// The decode grid's first workgroups (as many as the chip starts at once) keep
// the place their index gives them. Every later workgroup ("claimer") bumps one
// counter once with the hardware's wrapping increment,
//   old = *counter;  *counter = old >= limit ? 0 : old + 1;  return old,
// with limit = claimers - 1, and takes place ticket_place(old, claimers) among
// the late places. Whatever value the counter holds when a call starts:
//   - c0 <= limit: the claimers draw c0 .. limit, then 0 .. c0 - 1: every
//     place once, and the counter ends at c0 again (0 after a clean call);
//   - c0 > limit (left by a call of another size that did not finish its
//     claims): the first claimer draws c0 and resets the counter, the others
//     draw 0 .. claimers - 2, and the clamp below gives the first claimer the
//     one place left, claimers - 1.
// So each late place is taken exactly once for any start value, and a call
// never needs the counter cleared first.
//
// constexpr functions are usable on both the host and the device, so the host
// test of this rule compiles this very header.
#pragma once

#include <stdint.h>

namespace pkv {

constexpr uint32_t ticket_place(uint32_t ticket, uint32_t claimers) {
  return ticket < claimers ? ticket : claimers - 1u;
}

// What the wrapping increment stores (the rule above; host-side checks only).
constexpr uint32_t ticket_counter_next(uint32_t old, uint32_t limit) { return old >= limit ? 0u : old + 1u; }

}  // namespace pkv
