"""libattn: MI355X (gfx950) attention forward/backward behind a C ABI."""
