"""MI355X (gfx950) implementation of the Kalman Delta Network mixer recurrence."""
