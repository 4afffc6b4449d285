// Declarations shared by the host translation units of libwq.
#ifndef WQ_INTERNAL_H_
#define WQ_INTERNAL_H_

#include <cstdint>

#include "../../include/wq.h"

namespace wq {

uint16_t f64_to_f16_bits(double v);   // round to nearest even; +-inf past 65504
double f16_bits_to_f64(uint16_t h);
uint8_t e3m2_encode(double t);        // finite t -> 6-bit e3m2 code (ties to even, saturating)
uint8_t e2m1_encode(double t);        // finite t -> 4-bit e2m1 code (ties to even, saturating)

}  // namespace wq

#endif  // WQ_INTERNAL_H_
