// Internal helpers shared by the library's translation units: error
// reporting across the C ABI, the unit layout, and small utilities.
#pragma once
#include <cstdint>
#include <cstdio>
#include <exception>
#include <string>

#include "mt.h"

namespace mt {

void set_error(const char* fmt, ...);

struct Error : std::exception {
    int code;
    explicit Error(int c) : code(c) {}
};

// Raise a library error with a formatted message.
#define MT_FAIL(code, ...)            \
    do {                              \
        ::mt::set_error(__VA_ARGS__); \
        throw ::mt::Error(code);      \
    } while (0)

#define MT_CHECK_ARG(cond, ...)                      \
    do {                                             \
        if (!(cond)) MT_FAIL(MT_E_ARG, __VA_ARGS__); \
    } while (0)

// Wrap an ABI body: converts exceptions into return codes.
template <class F>
int guard(F&& f) {
    try {
        f();
        return MT_OK;
    } catch (const Error& e) {
        return e.code;
    } catch (const std::bad_alloc&) {
        set_error("host allocation failed");
        return MT_E_NOMEM;
    } catch (const std::exception& e) {
        set_error("unexpected error: %s", e.what());
        return MT_E_STATE;
    } catch (...) {
        set_error("unexpected non-standard exception");
        return MT_E_STATE;
    }
}

inline uint64_t round_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

// Validated layout of a unit (throws on bad config).
mt_unit_layout layout_of(const mt_model_cfg* cfg, int unit, uint32_t flags = 0);
void check_cfg(const mt_model_cfg* cfg);

}  // namespace mt
