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
uint8_t e2m2_encode(double t);        // finite t -> 5-bit e2m2 code (ties to even, saturating)

// The tiled prefill kernel (wq_prefill.hip). pf_takes: whether it runs `count` linears (N[i] x
// K[i]) of kernel code `code` at M rows of x, in one launch. The launches return a wq_status;
// arguments are checked by the caller.
bool pf_takes(int code, int64_t M, const int64_t* N, const int64_t* K, int count);
int pf_launch(int code, const uint16_t* x, const void* packed_w, const uint16_t* scales, const uint16_t* zeros,
              uint16_t* y, int64_t M, int64_t N, int64_t K, void* stream);
int pf_launch_grouped(int code, const wq_linear_item* items, int count, int64_t M, void* stream);

// A hipError_t from a launch -> WQ_OK, or WQ_ERR_DEVICE after keeping the error for
// wq_last_device_error (per thread).
int device_status(int hip_error);

}  // namespace wq

#endif  // WQ_INTERNAL_H_
